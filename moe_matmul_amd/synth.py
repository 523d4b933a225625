"""Seeded synthetic inputs for the NVFP4 block-scaled grouped GEMM.

This module draws raw bytes only. It decodes nothing, multiplies nothing and
knows nothing of where a scale sits inside the tiled scale tensor: it fills
whole buffers with random codes. Both the CPU oracle and the GPU path read
these same bytes.

Workloads (sizes from the grouped-GEMM task the pages solve; see the
``custom_kernel`` docstring on page 3, "kernelbot-nvfp4-group-gemm-499344"):

* ``A`` of group g: uint8 ``[l][m][k/2]``, two FP4 E2M1 codes per byte,
  K-major. Every byte is uniform over 0..255, so each nibble is uniform over
  the 16 codes.
* ``B``: uint8 ``[l][n][k/2]``, same distribution.
* ``SFA`` / ``SFB``: the tiled scale tensors, one E4M3 byte per 16 K-elements,
  padded to whole 128-row by 64-K atoms. Every byte of the buffer (padding
  included) is drawn uniformly from the 56 finite positive E4M3 codes whose
  unbiased exponent lies in [-3, 3] (biased exponent field 4..10, any
  mantissa), i.e. values in [0.125, 15].
* ``C``: fp16 ``[l][m][n]``, allocated by the caller.

For the two MoE workloads the first draw of the generator is the list of the
8 per-group ``m`` values, uniform over [40, 400].
"""
from __future__ import annotations

import numpy as np

# The 56 E4M3 codes (exponent field 4..10, any mantissa): positive and finite.
SCALE_CODES = np.array([(e << 3) | mnt for e in range(4, 11) for mnt in range(8)], dtype=np.uint8)
# The 7 of them with mantissa 0 (2^-3 .. 2^3): MX-compatible scales, for the
# power-of-two entry point's workloads.
POW2_SCALE_CODES = np.array([e << 3 for e in range(4, 11)], dtype=np.uint8)

# (name, per-group (m, n, k, l) or None when m is drawn, n, k)
WORKLOADS = {
    0: dict(name="g2_m128_n128_k256", shapes=[(128, 128, 256, 1)] * 2),
    1: dict(name="g4_m256_n512_k1024", shapes=[(256, 512, 1024, 1)] * 4),
    2: dict(name="g8_moe_mU40-400_n4096_k7168", groups=8, n=4096, k=7168),
    3: dict(name="g8_moe_down_mU40-400_n7168_k2048", groups=8, n=7168, k=2048),
    4: dict(name="g2_dense_4096x4096x8192_2048x7168x4096",
            shapes=[(4096, 4096, 8192, 1), (2048, 7168, 4096, 1)]),
}


def sf_buffer_bytes(rows: int, k: int, l: int = 1) -> int:
    """Size of one tiled scale tensor: whole atoms of 128 rows by 64 K-elements,
    4 scale bytes per row per atom."""
    return ((rows + 127) // 128) * 128 * ((k + 63) // 64) * 4 * l


def workload_shapes(index: int, seed: int | None = None) -> list[tuple[int, int, int, int]]:
    """Per-group (m, n, k, l) of a workload, with the drawn m list for the MoE ones."""
    w = WORKLOADS[index]
    if "shapes" in w:
        return list(w["shapes"])
    rng = np.random.default_rng(1000 + index if seed is None else seed)
    ms = rng.integers(40, 401, size=w["groups"])
    return [(int(m), w["n"], w["k"], 1) for m in ms]


def draw_group(rng: np.random.Generator, m: int, n: int, k: int, l: int = 1, scale_codes=SCALE_CODES) -> dict:
    """Random bytes of one group: packed A, packed B and the two scale buffers."""
    a = rng.integers(0, 256, size=(l, m, k // 2), dtype=np.uint8)
    b = rng.integers(0, 256, size=(l, n, k // 2), dtype=np.uint8)
    sfa = scale_codes[rng.integers(0, len(scale_codes), size=sf_buffer_bytes(m, k, l))]
    sfb = scale_codes[rng.integers(0, len(scale_codes), size=sf_buffer_bytes(n, k, l))]
    return dict(a=a, b=b, sfa=sfa, sfb=sfb)


def make_workload(index: int, seed: int | None = None,
                  scale_codes=SCALE_CODES) -> tuple[list[tuple[int, int, int, int]], list[dict]]:
    """Seeded workload ``index``: (problem_sizes, per-group byte arrays).
    ``scale_codes``: the pool the scale bytes are drawn from (POW2_SCALE_CODES
    for the power-of-two variant of a workload: same shapes, same m draw)."""
    rng = np.random.default_rng(1000 + index if seed is None else seed)
    w = WORKLOADS[index]
    if "shapes" in w:
        shapes = list(w["shapes"])
    else:
        ms = rng.integers(40, 401, size=w["groups"])
        shapes = [(int(m), w["n"], w["k"], 1) for m in ms]
    groups = [draw_group(rng, *s, scale_codes=np.asarray(scale_codes, dtype=np.uint8)) for s in shapes]
    return shapes, groups


def make_custom(shapes, seed: int, scale_codes: np.ndarray | None = None) -> list[dict]:
    """Random groups for arbitrary shapes (edge cases); optional scale code pool."""
    rng = np.random.default_rng(seed)
    pool = SCALE_CODES if scale_codes is None else np.asarray(scale_codes, dtype=np.uint8)
    out = []
    for (m, n, k, l) in shapes:
        a = rng.integers(0, 256, size=(l, m, k // 2), dtype=np.uint8)
        b = rng.integers(0, 256, size=(l, n, k // 2), dtype=np.uint8)
        sfa = pool[rng.integers(0, len(pool), size=sf_buffer_bytes(m, k, l))]
        sfb = pool[rng.integers(0, len(pool), size=sf_buffer_bytes(n, k, l))]
        out.append(dict(a=a, b=b, sfa=sfa, sfb=sfb))
    return out


# The super-batch of the pages: the groups of 15 benchmark calls (each with up
# to 8 groups, each call with its own data) merged into one launch.
SUPER_BATCH_COPIES = 15


def make_super_batch(index: int, copies: int = SUPER_BATCH_COPIES):
    """``copies`` calls of workload ``index`` as one grouped problem: the same
    per-group shapes repeated, each copy's bytes drawn from its own seed."""
    shapes = workload_shapes(index)
    all_shapes, groups = [], []
    for c in range(copies):
        rng = np.random.default_rng(1000 + index + 7919 * (c + 1))
        all_shapes += shapes
        groups += [draw_group(rng, *s) for s in shapes]
    return all_shapes, groups
