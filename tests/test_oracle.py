"""Pins of the CPU oracle against things other than itself (CPU only).

* E4M3FN decode: all 256 codes against torch's float8_e4m3fn (a library routine).
* E2M1 decode: the format's bit-field definition (bias 1, subnormal at exponent 0).
* Tiled scale layout: a small evaluator of CuTe layout algebra applied to the atom
  ((32, 4), (16, 4)) : ((16, 4), (0, 1)) tiled over (m, k, l) in the order (2, 1, 3),
  as built in ``kernel`` of submission 385043 and ``init_tensormaps_kernel`` of
  submission 499344 (kernelindex.com, kernelbot nvfp4 group gemm).
* Accumulation: an independent integer oracle (bit-field decode, int64 sums).
* Whole oracle: hand-worked cases (tests/golden/hand_cases.json), exact-rational
  brute force, unit-scale quarter-integrality, and invariants (scale doubling,
  transposition, negation, group independence, nibble-order invariance).
* Rounding: an exact-rational round-to-nearest-even into fp16.
* Mutations: plausible mistakes planted in the oracle must each break a pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.nvfp4_oracle as O
from moe_matmul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ----------------------------------------------------------------------------
# Independent helpers (no oracle code)
# ----------------------------------------------------------------------------

def e2m1_twice(code: int) -> int:
    """2 * value of an E2M1 code, from its bit fields."""
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = m if e == 0 else (2 + m) << (e - 1)
    return -mag if s else mag


def e4m3_times512(code: int) -> int:
    """512 * value of a finite E4M3FN code, from its bit fields."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    mag = m if e == 0 else (8 + m) << (e - 1)
    return -mag if s else mag


E2M1_TWICE = np.array([e2m1_twice(c) for c in range(16)], dtype=np.int64)
E4M3_X512 = np.array([e4m3_times512(c) if (c & 0x7F) != 0x7F else 0 for c in range(256)], dtype=np.int64)


def rne_fp16_bits(x: Fraction) -> int:
    """Exact rational -> fp16 bit pattern, round to nearest, ties to even."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)
    q = Fraction(2) ** (e - 10)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v >= 65536:
        return sign | 0x7C00
    if v < Fraction(2) ** -14:
        return sign | int(v / Fraction(2) ** -24)
    E = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** E > v:
        E -= 1
    while Fraction(2) ** (E + 1) <= v:
        E += 1
    mant = (v / Fraction(2) ** E - 1) * 1024
    assert mant.denominator == 1
    return sign | ((E + 15) << 10) | int(mant)


def fp16_bits(x) -> int:
    return int(np.asarray([x], dtype=np.float16).view(np.uint16)[0])


# --- a small evaluator of CuTe layout algebra (shape/stride trees, colexicographic) ---

def _size(shape):
    if isinstance(shape, tuple):
        return math.prod(_size(s) for s in shape)
    return shape


def _crd2idx(c, shape, stride):
    """Map a 1-D coordinate (int or int array) through a hierarchical layout mode."""
    if isinstance(shape, tuple):
        idx = 0
        for i, (s, d) in enumerate(zip(shape, stride)):
            if i == len(shape) - 1:
                idx = idx + _crd2idx(c, s, d)
            else:
                sz = _size(s)
                idx = idx + _crd2idx(c % sz, s, d)
                c = c // sz
        return idx
    return c * stride


def _ordered_strides(shape, order):
    """Compact strides where the mode with the smallest order value is fastest."""
    strides = [0] * len(shape)
    cur = 1
    for i in sorted(range(len(shape)), key=lambda i: order[i]):
        strides[i] = cur
        cur *= shape[i]
    return strides


def cute_tile_to_shape(atom_shape, atom_stride, target, order):
    """Blocked product of the atom with an ordered tiler that covers ``target``."""
    modes_shape = list(atom_shape) + [1] * (len(target) - len(atom_shape))
    modes_stride = list(atom_stride) + [0] * (len(target) - len(atom_stride))
    # cosize of the atom: one past its largest image
    dom = _size(tuple(modes_shape))
    atom_img = 0
    coords = np.arange(dom)
    c = coords.copy()
    for s, d in zip(modes_shape, modes_stride):
        sz = _size(s)
        atom_img = atom_img + _crd2idx(c % sz, s, d)
        c = c // sz
    cosize = int(np.max(atom_img)) + 1
    prod_shape = [-(-target[i] // _size(modes_shape[i])) for i in range(len(target))]
    tstr = [s * cosize for s in _ordered_strides(prod_shape, order)]
    return [((modes_shape[i], prod_shape[i]), (modes_stride[i], tstr[i])) for i in range(len(target))]


def cute_sf_offset(r, kk, li, rows, k, l):
    """Offset of the scale of row r, K-element kk, batch li, via the evaluator."""
    layout = cute_tile_to_shape(((32, 4), (16, 4)), ((16, 4), (0, 1)), (rows, k, l), (2, 1, 3))
    return sum(_crd2idx(c, s, d) for c, (s, d) in zip((r, kk, li), layout))


def int_oracle(m, n, k, a, b, sfa, sfb, rows=None):
    """C * 2**20 as exact integers: bit-field decode, CuTe-evaluator scale gather."""
    a = np.asarray(a, np.uint8).reshape(m, k // 2)
    b = np.asarray(b, np.uint8).reshape(n, k // 2)

    def operand(p, sf, nrows, sel):
        codes = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[0], k)[sel]
        vals = E2M1_TWICE[codes]
        r = np.asarray(sel)[:, None]
        kk = (np.arange(k // 16) * 16)[None, :]
        off = cute_sf_offset(r, kk, 0, nrows, k, 1)
        sc = E4M3_X512[np.asarray(sf, np.uint8)[off]]
        return vals * np.repeat(sc, 16, axis=1)

    sel = np.arange(m) if rows is None else np.asarray(rows)
    ai = operand(a, sfa, m, sel)
    bi = operand(b, sfb, n, np.arange(n))
    return ai @ bi.T


def build_single(case):
    """Byte buffers of a 1x1xk hand case."""
    def expand(spec):
        out = []
        for tok in spec.split(","):
            if "*" in tok:
                v, c = tok.split("*")
                out += [int(v)] * int(c)
            else:
                out.append(int(tok))
        return out

    k = case["k"]
    ac, bc = expand(case["a"]), expand(case["b"])
    assert len(ac) == k and len(bc) == k
    pack = lambda codes: np.array([codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(k // 2)], np.uint8)
    nbytes = synth.sf_buffer_bytes(1, k)
    sfa = np.zeros(nbytes, np.uint8)
    sfb = np.zeros(nbytes, np.uint8)
    for kb, (x, y) in enumerate(zip(case["sfa"], case["sfb"])):
        off = cute_sf_offset(0, kb * 16, 0, 1, k, 1)
        sfa[off], sfb[off] = x, y
    return dict(a=pack(ac), b=pack(bc), sfa=sfa, sfb=sfb)


# ----------------------------------------------------------------------------
# Decode pins
# ----------------------------------------------------------------------------

def test_e2m1_table_matches_bit_fields():
    vals = O.decode_e2m1(np.arange(16))
    for c in range(16):
        assert vals[c] == e2m1_twice(c) / 2
        assert math.copysign(1.0, vals[c]) == (-1.0 if c & 8 else 1.0)
    assert sorted(set(np.abs(vals).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3fn_matches_torch_all_codes():
    ours = O.decode_e4m3fn(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert O.decode_e4m3fn(np.array([0x7E]))[0] == 448.0
    assert O.decode_e4m3fn(np.array([0x01]))[0] == 2.0 ** -9


def test_e4m3_bit_field_integer_decode_agrees():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert O.decode_e4m3fn(np.array([c]))[0] * 512 == e4m3_times512(c)


def test_config_scale_codes_span_exponents():
    vals = O.decode_e4m3fn(synth.SCALE_CODES)
    assert len(set(synth.SCALE_CODES.tolist())) == 56
    assert vals.min() == 0.125 and vals.max() == 15.0
    assert np.all(np.floor(np.log2(vals)) >= -3) and np.all(np.floor(np.log2(vals)) <= 3)


# ----------------------------------------------------------------------------
# Scale layout pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,k,l", [(1, 64, 1), (128, 256, 1), (300, 512, 1), (129, 192, 2), (1, 32, 1),
                                      (129, 96, 2), (300, 160, 1)])
def test_sf_offset_matches_cute_layout(rows, k, l):
    mt = -(-rows // 128) * 128
    r = np.arange(mt)[:, None]
    kk = np.arange(k)[None, :]
    for li in range(l):
        ref = cute_sf_offset(r, kk, li, rows, k, l)
        ours = O.sf_offset(r, kk // 16, rows, k, li)
        assert np.array_equal(np.broadcast_to(ref, ours.shape), ours)


def test_sf_layout_is_bijective_and_tiles_are_contiguous():
    rows, k = 300, 512
    mt, kt = 3, 8
    r = np.arange(mt * 128)[:, None]
    kb = np.arange(k // 16)[None, :]
    off = O.sf_offset(r, kb, rows, k).reshape(-1)
    assert sorted(off.tolist()) == list(range(synth.sf_buffer_bytes(rows, k)))
    # a 128-row by 256-K tile is one contiguous 2 KiB span
    for tm in range(mt):
        for tk in range(kt // 4):
            o = O.sf_offset(np.arange(tm * 128, tm * 128 + 128)[:, None],
                            np.arange(tk * 16, tk * 16 + 16)[None, :], rows, k)
            assert o.min() == (tm * kt + tk * 4) * 512 and o.max() == o.min() + 2047
            assert len(set(o.reshape(-1).tolist())) == 2048


# ----------------------------------------------------------------------------
# Whole-oracle pins
# ----------------------------------------------------------------------------

def _hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    grp = build_single(case)
    out = O.grouped_gemm([(1, 1, case["k"], 1)], [grp])[0]
    exact = Fraction(case["exact"])
    assert Fraction(out["c64"][0, 0, 0]) == exact
    assert fp16_bits(out["c16"][0, 0, 0]) == int(case["fp16_bits"], 16)
    assert rne_fp16_bits(exact) == int(case["fp16_bits"], 16)


def test_unit_scales_give_quarter_integers():
    (grp,) = synth.make_custom([(64, 48, 256, 1)], seed=7, scale_codes=[0x38])
    out = O.grouped_gemm([(64, 48, 256, 1)], [grp])[0]
    q = out["c64"] * 4
    assert np.array_equal(q, np.round(q))
    ref = int_oracle(64, 48, 256, grp["a"], grp["b"], grp["sfa"], grp["sfb"])
    assert np.array_equal(out["c64"][0] * 2 ** 20, ref.astype(np.float64))


def test_bruteforce_equal_element_blocks():
    """Every (a code, b code) pair times every pair of workload scales on 1x1x16
    blocks whose 16 elements are equal: C = 16 * a * sa * b * sb exactly."""
    codes = np.arange(16)
    sc = synth.SCALE_CODES
    m = n = 16 * len(sc)
    # row i: code i % 16 everywhere, scale sc[i // 16]
    rc, rs = codes[np.arange(m) % 16], sc[np.arange(m) // 16]
    a = np.repeat((rc | (rc << 4)).astype(np.uint8)[:, None], 8, axis=1)
    nbytes = synth.sf_buffer_bytes(m, 64)
    sfa = np.zeros(nbytes, np.uint8)
    sfa[O.sf_offset(np.arange(m), 0, m, 64)] = rs
    # k = 64 with blocks 1..3 zero
    a64 = np.zeros((m, 32), np.uint8)
    a64[:, :8] = a
    out = O.grouped_gemm([(m, n, 64, 1)], [dict(a=a64, b=a64, sfa=sfa, sfb=sfa)])[0]
    exact = 16 * np.outer(E2M1_TWICE[rc] * E4M3_X512[rs], E2M1_TWICE[rc] * E4M3_X512[rs])
    assert np.array_equal(out["c64"][0] * 2 ** 20, exact.astype(np.float64))
    # a sample checked bit-for-bit through exact rational rounding
    rng = np.random.default_rng(3)
    for i, j in rng.integers(0, m, size=(300, 2)):
        fr = Fraction(int(exact[i, j]), 2 ** 20)
        assert fp16_bits(out["c16"][0, i, j]) == rne_fp16_bits(fr)


def test_bruteforce_random_blocks_fraction():
    rng = np.random.default_rng(11)
    for trial in range(60):
        k = 64
        a_codes = rng.integers(0, 16, k)
        b_codes = rng.integers(0, 16, k)
        sa = rng.choice(synth.SCALE_CODES, 4) if trial % 2 else rng.integers(0, 0x7F, 4)
        sb = rng.choice(synth.SCALE_CODES, 4) if trial % 2 else rng.integers(0, 0x7F, 4)
        case = dict(k=k, a=",".join(map(str, a_codes)), b=",".join(map(str, b_codes)),
                    sfa=[int(x) for x in sa], sfb=[int(x) for x in sb])
        grp = build_single(case)
        out = O.grouped_gemm([(1, 1, k, 1)], [grp])[0]
        exact = sum(Fraction(e2m1_twice(int(a_codes[i])), 2) * Fraction(e4m3_times512(int(sa[i // 16])), 512)
                    * Fraction(e2m1_twice(int(b_codes[i])), 2) * Fraction(e4m3_times512(int(sb[i // 16])), 512)
                    for i in range(k))
        assert Fraction(out["c64"][0, 0, 0]) == exact
        assert fp16_bits(out["c16"][0, 0, 0]) == rne_fp16_bits(exact)


def test_fp16_rounding_boundaries():
    cases = [2049, Fraction(20490000001, 10000000), 2051, Fraction(655199, 10), 65520,
             Fraction(1, 2 ** 25), Fraction(3, 2 ** 26), -65520, Fraction(65504), Fraction(-1, 3)]
    for v in cases:
        got = fp16_bits(O.round_to_fp16(np.array([float(v)]))[0])
        # float(v) is exact for all but 2049.0000001 / 6551.99 / -1/3, whose float64
        # neighbourhood is far from any fp16 tie.
        assert got == rne_fp16_bits(Fraction(float(v))), v


def test_integer_oracle_agrees_on_small_workloads():
    for idx in (0, 1):
        shapes, groups = synth.make_workload(idx)
        outs = O.grouped_gemm(shapes, groups)
        for (m, n, k, l), grp, out in zip(shapes, groups, outs):
            assert out["exact"]
            ref = int_oracle(m, n, k, grp["a"], grp["b"], grp["sfa"], grp["sfb"])
            assert np.array_equal(out["c64"][0] * 2 ** 20, ref.astype(np.float64))


@pytest.mark.parametrize("idx", [2, 3])
def test_integer_oracle_agrees_on_sampled_rows(idx):
    shapes, groups = synth.make_workload(idx)
    rng = np.random.default_rng(5)
    for g in (0, len(shapes) - 1):
        m, n, k, l = shapes[g]
        rows = np.sort(rng.choice(m, 3, replace=False))
        out = O.grouped_gemm([shapes[g]], [groups[g]], rows=[rows])[0]
        ref = int_oracle(m, n, k, groups[g]["a"], groups[g]["b"], groups[g]["sfa"], groups[g]["sfb"], rows=rows)
        assert out["exact"]
        assert np.array_equal(out["c64"][0] * 2 ** 20, ref.astype(np.float64))


def test_workload_m_lists():
    assert [s[0] for s in synth.workload_shapes(2)] == [258, 177, 320, 168, 362, 309, 260, 180]
    assert [s[0] for s in synth.workload_shapes(3)] == [147, 107, 250, 132, 142, 218, 353, 278]
    shapes, _ = synth.make_workload(0)
    assert shapes == [(128, 128, 256, 1)] * 2


def _rand_group(m, n, k, seed):
    (g,) = synth.make_custom([(m, n, k, 1)], seed=seed)
    return g


def test_scale_doubling_adds_exactly_that_block():
    m, n, k = 40, 24, 128
    grp = _rand_group(m, n, k, 21)
    base = O.grouped_gemm([(m, n, k, 1)], [grp])[0]["c64"][0]
    r, kb = 13, 5
    off = cute_sf_offset(r, kb * 16, 0, m, k, 1)
    code = int(grp["sfa"][off])
    assert ((code >> 3) & 15) < 14
    g2 = dict(grp, sfa=grp["sfa"].copy())
    g2["sfa"][off] = code + 8          # exponent + 1: the scale doubles
    new = O.grouped_gemm([(m, n, k, 1)], [g2])[0]["c64"][0]
    diff = new - base
    assert np.all(diff[np.arange(m) != r] == 0)
    # the block's contribution, summed independently in integers
    codes_a = np.stack([grp["a"][0] & 15, grp["a"][0] >> 4], -1).reshape(m, k)[r, kb * 16:(kb + 1) * 16]
    codes_b = np.stack([grp["b"][0] & 15, grp["b"][0] >> 4], -1).reshape(n, k)[:, kb * 16:(kb + 1) * 16]
    sb = np.array([E4M3_X512[grp["sfb"][cute_sf_offset(j, kb * 16, 0, n, k, 1)]] for j in range(n)])
    contrib = (E2M1_TWICE[codes_b] @ E2M1_TWICE[codes_a]) * E4M3_X512[code] * sb
    assert np.array_equal(diff[r] * 2 ** 20, contrib.astype(np.float64))


def test_transpose_symmetry():
    m, n, k = 33, 70, 192
    ga = _rand_group(m, n, k, 1)
    gb = _rand_group(n, m, k, 2)
    g1 = dict(a=ga["a"], b=gb["a"], sfa=ga["sfa"], sfb=gb["sfa"])
    g2 = dict(a=gb["a"], b=ga["a"], sfa=gb["sfa"], sfb=ga["sfa"])
    c1 = O.grouped_gemm([(m, n, k, 1)], [g1])[0]["c64"][0]
    c2 = O.grouped_gemm([(n, m, k, 1)], [g2])[0]["c64"][0]
    assert np.array_equal(c1, c2.T)


def test_negating_a_negates_c():
    m, n, k = 20, 30, 64
    g = _rand_group(m, n, k, 4)
    gn = dict(g, a=g["a"] ^ np.uint8(0x88))
    c = O.grouped_gemm([(m, n, k, 1)], [g])[0]["c64"][0]
    cn = O.grouped_gemm([(m, n, k, 1)], [gn])[0]["c64"][0]
    assert np.array_equal(c, -cn)


@pytest.mark.parametrize("k", [32, 96, 160])
def test_half_atom_k_is_the_truncated_sum(k):
    """k % 64 == 32: the result equals the integer oracle's (CuTe-evaluator
    gather) and the oracle's own result for k + 32 with the extra 32 codes of
    every row zero (their scales are the bytes of the last atom's unused half,
    finite codes in these buffers)."""
    m, n = 37, 24
    grp = _rand_group(m, n, k, 96 + k)
    out = O.grouped_gemm([(m, n, k, 1)], [grp])[0]
    ref = int_oracle(m, n, k, grp["a"], grp["b"], grp["sfa"], grp["sfb"])
    assert np.array_equal(out["c64"][0] * 2 ** 20, ref.astype(np.float64))
    k2 = k + 32
    assert synth.sf_buffer_bytes(m, k2) == synth.sf_buffer_bytes(m, k)  # same atoms, now fully used
    ext = {}
    for key, rows in (("a", m), ("b", n)):
        x = np.zeros((1, rows, k2 // 2), np.uint8)
        x[0, :, : k // 2] = grp[key][0]
        ext[key] = x
    for key in ("sfa", "sfb"):
        ext[key] = grp[key].copy()
    longer = O.grouped_gemm([(m, n, k2, 1)], [ext])[0]
    assert np.array_equal(longer["c64"], out["c64"])


def test_groups_are_independent():
    shapes = [(17, 40, 64, 1), (130, 8, 128, 1), (5, 64, 256, 1)]
    groups = synth.make_custom(shapes, seed=9)
    together = O.grouped_gemm(shapes, groups)
    for s, g, t in zip(shapes, groups, together):
        alone = O.grouped_gemm([s], [g])[0]
        assert np.array_equal(alone["c64"], t["c64"])


def test_nibble_order_is_unobservable():
    m, n, k = 12, 9, 128
    g = _rand_group(m, n, k, 8)
    swap = lambda x: ((x & 15) << 4) | (x >> 4)
    gs = dict(g, a=swap(g["a"]), b=swap(g["b"]))
    c = O.grouped_gemm([(m, n, k, 1)], [g])[0]["c64"]
    cs = O.grouped_gemm([(m, n, k, 1)], [gs])[0]["c64"]
    assert np.array_equal(c, cs)


def test_empty_dims():
    for (m, n, k) in [(0, 8, 64), (8, 0, 64), (4, 8, 0)]:
        grp = dict(a=np.zeros((1, m, k // 2), np.uint8), b=np.zeros((1, n, k // 2), np.uint8),
                   sfa=np.zeros(synth.sf_buffer_bytes(m, k), np.uint8),
                   sfb=np.zeros(synth.sf_buffer_bytes(n, k), np.uint8))
        out = O.grouped_gemm([(m, n, k, 1)], [grp])[0]
        assert out["c64"].shape == (1, m, n) and np.all(out["c64"] == 0)


def test_tolerance_rule():
    ref = np.array([2048.0, 65504.0, np.inf, 1.0, 0.0, 100.0], np.float16)
    s = np.array([0.0, 0.0, 0.0, 0.0, 1e4, 0.0])
    ok = np.array([2052.0, np.inf, 65504.0, 1.0 + 2 * 2 ** -10, 0.1, 100.0], np.float16)
    assert not O.tolerance_violations(ok, ref, s).any()
    bad = np.array([2056.0, -np.inf, np.nan, 1.0 + 3 * 2 ** -10, 0.2, np.nan], np.float16)
    assert O.tolerance_violations(bad, ref, s).all()


# ----------------------------------------------------------------------------
# Mutations planted in the oracle (CPU) must each break at least one pin
# ----------------------------------------------------------------------------

def _pin_battery():
    """Run the cheap pins; return the names of those that fail."""
    failed = []
    for case in _hand_cases():
        try:
            test_hand_cases(case)
        except AssertionError:
            failed.append(case["name"])
    for name, fn in [("unit", test_unit_scales_give_quarter_integers),
                     ("brute", test_bruteforce_random_blocks_fraction),
                     ("layout", lambda: test_sf_offset_matches_cute_layout(300, 512, 1)),
                     ("doubling", test_scale_doubling_adds_exactly_that_block),
                     ("rounding", test_fp16_rounding_boundaries)]:
        try:
            fn()
        except (AssertionError, IndexError, ValueError):
            failed.append(name)
    return failed


def test_pin_battery_passes_unmutated():
    assert _pin_battery() == []


_orig_sf_offset = O.sf_offset
_orig_dequantize = O.dequantize
_orig_gather = O.gather_scales
_orig_e4m3 = O.decode_e4m3fn

MUTATIONS = {
    "e2m1_wrong_entry": ("E2M1_VALUES", np.where(np.arange(16) == 5, 2.5, O.E2M1_VALUES)),
    "e2m1_lost_sign": ("E2M1_VALUES", np.abs(O.E2M1_VALUES)),
    "e4m3_bias_8": ("decode_e4m3fn", lambda c: _orig_e4m3(c) / 2),
    "e4m3_subnormal_off": ("decode_e4m3fn", lambda c: np.where((np.asarray(c) >> 3) & 15 == 0,
                                                                _orig_e4m3(c) / 2,
                                                                _orig_e4m3(c))),
    "sf_atom_row_major": ("sf_offset", lambda r, kb, rows, k, li=0:
                          _orig_sf_offset(r, kb, rows, k, li)
                          - (np.asarray(r) % 32) * 16 - ((np.asarray(r) // 32) % 4) * 4
                          + (np.asarray(r) % 128) * 4),
    "sf_block_off_by_one": ("gather_scales", lambda t, rows, k, li=0:
                            np.roll(_orig_gather(t, rows, k, li), 1, axis=1)),
    "dropped_last_block": ("dequantize", lambda p, sf, rows, k, li=0, row_subset=None:
                           _orig_dequantize(p, sf, rows, k, li, row_subset)
                           * (np.arange(k) < k - 16)[None, :]),
    "double_rounding_fp32": ("round_to_fp16", lambda x: np.asarray(x).astype(np.float32).astype(np.float16)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(O, attr, value)
    failed = _pin_battery()
    assert failed, f"mutation {name} went unnoticed"
