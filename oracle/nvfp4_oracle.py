"""CPU oracle for the NVFP4 block-scaled grouped GEMM.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
CPU-baseline leg of the benchmark may import this module. The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path.

What it computes (the plain definition, rounded once):

    C_g[m, n] = sum_k (a_g[m, k] * sfa_g[m, k // 16]) * (b_g[n, k] * sfb_g[n, k // 16])

Sources, all on the kernelindex.com pages "kernelbot nvfp4 group gemm":

* The contraction: the mainloop comment of submission 499344 states that the
  accumulator gathers A times SFA times B times SFB; submission 506336's
  ``my_kernel`` builds the block-scaled MMA from the FP4 operand type and the
  FP8 scale type.
* Formats: operands ``Float4E2M1FN``, scales ``Float8E4M3FN``, one scale per
  16 K-elements (``sf_vec_size``), fp16 output (module constants of all three
  submissions).
* Operand layouts: A is (m, k, l) with strides (k, 1, m*k) and B is (n, k, l)
  with strides (k, 1, n*k), i.e. K-major; C is (m, n, l) row-major
  (``kernel`` of submission 385043 and of submission 506336).
* Scale layout: the atom of shape ((32, 4), (16, 4)) and stride
  ((16, 4), (0, 1)) tiled over (m, k, l) in the order (2, 1, 3) (``kernel`` of
  submission 385043; ``init_tensormaps_kernel`` of submission 499344).
* Interface: ``custom_kernel`` docstring of submission 499344.

Readings where the pages are silent or disagree:

* E4M3 variant: the code uses ``Float8E4M3FN`` while the docstring of
  submission 499344 says ``float8_e4m3fnuz``; the oracle decodes E4M3FN
  (bias 7, no infinities, 0x7F and 0xFF are NaN, largest 448).
* Nibble order: the low nibble of byte j holds element 2j. (C does not depend
  on this as long as A and B agree, because both elements of a byte lie in one
  16-element block.)
* Rounding: float64 sum rounded once to fp16, round-to-nearest-even,
  overflow to +-inf.
* k = 0 gives C = 0 (the empty sum).

Accumulation is exact: every term is an integer multiple of a power of two
fixed by the smallest scales, and the oracle checks that the largest possible
partial sum stays below 2**53 of those units, so no summation order can round.
If that check fails (tiny subnormal scales with huge k), ``exact`` is False
and the float64 result carries ordinary rounding error, far below the
tolerance.
"""
from __future__ import annotations

import math

import numpy as np

# E2M1 values by 4-bit code: bit 3 is the sign, bits 2..1 the exponent
# (bias 1), bit 0 the mantissa; exponent 0 is subnormal (0 or 0.5).
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)

SF_VEC = 16          # K-elements per scale (sf_vec_size)
ATOM_ROWS = 128      # rows of one scale atom: 32 x 4
ATOM_KBLOCKS = 4     # scale blocks (of 16 K) of one atom
ATOM_BYTES = 512


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows, k/2] -> uint8 codes [rows, k]; low nibble is the even element."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    return codes


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 code -> float64, through the 16-entry value table."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8)]


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN byte -> float64, exactly, from its bit fields.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    Exponent 0 is subnormal: mantissa/8 * 2**-6. 0x7F and 0xFF are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = (1.0 + mant / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    sub = mant / 8.0 * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def sf_offset(r, kb, rows: int, k: int, li=0):
    """Byte offset of the scale of row ``r``, 16-block ``kb``, batch ``li``.

    The atom ((32, 4), (16, 4)) : ((16, 4), (0, 1)) sends row r to
    16*(r % 32) + 4*((r // 32) % 4) and K-element kk to (kk // 16) % 4; the 16
    elements of a block share one byte (stride 0). Tiling in the order
    (2, 1, 3) repeats atoms along K first (512 bytes apart), then along M
    (Kt*512 apart), then along l.
    """
    kt = (k + 63) // 64
    mt = (rows + 127) // 128
    r = np.asarray(r, dtype=np.int64)
    kb = np.asarray(kb, dtype=np.int64)
    return (li * mt * kt * ATOM_BYTES
            + (r // ATOM_ROWS) * kt * ATOM_BYTES
            + (kb // ATOM_KBLOCKS) * ATOM_BYTES
            + (r % 32) * 16 + ((r // 32) % 4) * 4 + (kb % ATOM_KBLOCKS))


def gather_scales(tiled: np.ndarray, rows: int, k: int, li: int = 0) -> np.ndarray:
    """Tiled scale bytes -> logical uint8 [rows, k/16] for batch ``li``."""
    tiled = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    r = np.arange(rows)[:, None]
    kb = np.arange(k // SF_VEC)[None, :]
    return tiled[sf_offset(r, kb, rows, k, li)]


def dequantize(packed: np.ndarray, tiled_sf: np.ndarray, rows: int, k: int, li: int = 0,
               row_subset=None) -> np.ndarray:
    """Operand value a * sf as float64 [rows, k] (exact)."""
    vals = decode_e2m1(unpack_fp4(packed))                     # [rows, k]
    sf = decode_e4m3fn(gather_scales(tiled_sf, rows, k, li))   # [rows, k/16]
    if row_subset is not None:
        vals, sf = vals[row_subset], sf[row_subset]
    return vals * np.repeat(sf, SF_VEC, axis=1)


def _granule_exponent(tiled_sf: np.ndarray, rows: int, k: int, li: int) -> int:
    """Exponent q such that every a*sf of this operand is a multiple of 2**q."""
    codes = gather_scales(tiled_sf, rows, k, li).reshape(-1)
    if codes.size == 0:
        return 0
    e = (codes.astype(np.int64) >> 3) & 0xF
    # a normal scale 2**(e-7) * (8+M)/8 is a multiple of 2**(e-10); a subnormal
    # one of 2**-9; an E2M1 value is a multiple of 2**-1.
    q_scale = np.where(e == 0, -9, e - 10)
    return int(q_scale.min()) - 1


def round_to_fp16(x64: np.ndarray) -> np.ndarray:
    """float64 -> fp16, rounded once to nearest-even (numpy rounds directly
    from float64; overflow gives +-inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float16)


def gemm_group(m: int, n: int, k: int, l: int, a, b, sfa, sfb, rows=None) -> dict:
    """One group: C64 (exact float64), C16 (rounded) and S = sum_k |terms|.

    ``rows`` optionally restricts the computation to a subset of output rows.
    Arrays are [l][rows][n].
    """
    a = np.asarray(a, dtype=np.uint8).reshape(l, m, k // 2)
    b = np.asarray(b, dtype=np.uint8).reshape(l, n, k // 2)
    sel = np.arange(m) if rows is None else np.asarray(rows)
    c64 = np.zeros((l, len(sel), n))
    s = np.zeros((l, len(sel), n))
    exact = True
    for li in range(l):
        if k == 0 or m == 0 or n == 0:
            continue
        ad = dequantize(a[li], sfa, m, k, li, row_subset=sel)
        bd = dequantize(b[li], sfb, n, k, li)
        if np.isnan(ad).any() or np.isnan(bd).any():
            exact = False
        c64[li] = ad @ bd.T
        s[li] = np.abs(ad) @ np.abs(bd).T
        q = _granule_exponent(sfa, m, k, li) + _granule_exponent(sfb, n, k, li)
        smax = np.nanmax(s[li]) if s[li].size else 0.0
        if not smax < math.ldexp(1.0, 53 + q):
            exact = False
    return dict(c64=c64, c16=round_to_fp16(c64), s=s, exact=exact)


def grouped_gemm(problem_sizes, groups, rows=None) -> list[dict]:
    """All groups; ``groups[g]`` holds byte arrays a, b, sfa, sfb.

    ``rows`` is None or a list (per group) of row subsets.
    """
    out = []
    for g, (m, n, k, l) in enumerate(problem_sizes):
        grp = groups[g]
        out.append(gemm_group(m, n, k, l, grp["a"], grp["b"], grp["sfa"], grp["sfb"],
                              None if rows is None else rows[g]))
    return out


def fp16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of fp16 numbers at |x|: 2**(floor(log2|x|) - 10) for normal |x|,
    2**-24 below 2**-14; |x| >= 65536 (an infinity mapped there) gets 32."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.where(ax >= 2.0 ** -14, np.ldexp(1.0, (e - 10).astype(np.int64)), 2.0 ** -24)
    return np.where(ax >= 65536.0, 32.0, ulp)


def tolerance_violations(c_gpu16: np.ndarray, c_ref16: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Boolean mask of elements that break |C - C_ref| <= 2 ulp16(C_ref) + 1e-5 S.

    Infinities count as +-65536 (so 65504 against +inf differs by one ulp);
    a NaN on either side is always a violation.
    """
    g = np.asarray(c_gpu16, dtype=np.float64)
    r = np.asarray(c_ref16, dtype=np.float64)
    nan = np.isnan(g) | np.isnan(r)
    g = np.where(np.isinf(g), np.sign(g) * 65536.0, g)
    r = np.where(np.isinf(r), np.sign(r) * 65536.0, r)
    with np.errstate(invalid="ignore"):
        bad = np.abs(g - r) > 2.0 * fp16_ulp(r) + 1e-5 * np.asarray(s, dtype=np.float64)
    return bad | nan
