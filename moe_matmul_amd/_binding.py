"""ctypes binding of the C ABI in include/nvfp4_grouped_gemm.h.

Argument marshalling only: every step of the computation runs in the HIP
library. The names mirror the C entry points. The library must have been
built (``python -m moe_matmul_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_grouped_gemm.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID = -1
NVFP4_ERR_MISALIGNED = -2
NVFP4_ERR_HIP = -3
NVFP4_ERR_CONFIG = -4
NVFP4_ERR_WORKSPACE = -5
NVFP4_MAX_GROUPS = 8
NVFP4_SCRATCH_BYTES = (32 << 20) + 65536
NVFP4_MAX_DEVICE_GROUPS = 512

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what} failed: {code} ({nvfp4_error_string(code)})"
                         + (f", hip error {nvfp4_last_hip_error()}" if code == NVFP4_ERR_HIP else ""))


def load_library() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m moe_matmul_amd.build` "
                          "(the NVFP4 grouped GEMM has no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    ip = ctypes.POINTER(ctypes.c_int)
    sig = {
        "nvfp4_grouped_gemm": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_void_p]),
        "nvfp4_grouped_gemm_config": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]),
        "nvfp4_grouped_gemm_validate": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int]),
        "nvfp4_num_tile_configs": (ctypes.c_int, []),
        "nvfp4_tile_config_info": (ctypes.c_int, [ctypes.c_int, ip, ip, ip, ip]),
        "nvfp4_select_tile_config": (ctypes.c_int, [i32p, ctypes.c_int, ctypes.c_int]),
        "nvfp4_launch_geometry": (ctypes.c_int, [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 i64p, ip, ip, ctypes.POINTER(ctypes.c_size_t)]),
        "nvfp4_splits_k_over_waves": (ctypes.c_int, [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "nvfp4_grouped_gemm_ex": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
        "nvfp4_grouped_gemm_scratch": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_void_p]),
        "nvfp4_grouped_gemm_stages": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_void_p,
                                                     ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_void_p]),
        "nvfp4_grouped_gemm_pow2": (ctypes.c_int, [i32p, u64p, u64p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
        "nvfp4_grouped_gemm_device": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
        "nvfp4_device_group_tiles": (ctypes.c_int64, [i32p, u64p, ctypes.c_int]),
        "nvfp4_workspace_bytes": (ctypes.c_size_t, [i32p, ctypes.c_int, ctypes.c_int]),
        "nvfp4_split_plan": (ctypes.c_int, [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p, ctypes.c_int]),
        "nvfp4_sf_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "nvfp4_last_hip_error": (ctypes.c_int, []),
        "nvfp4_error_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _sizes(problem_sizes):
    if isinstance(problem_sizes, ctypes.Array) and problem_sizes._type_ is ctypes.c_int32:
        return problem_sizes, len(problem_sizes) // 4  # already marshalled (see prepare)
    flat = [int(v) for row in problem_sizes for v in row]
    return (ctypes.c_int32 * max(len(flat), 1))(*flat), len(flat) // 4


def _u64(rows, width):
    if isinstance(rows, ctypes.Array) and rows._type_ is ctypes.c_uint64:
        return rows
    flat = [int(v) for row in rows for v in row]
    if len(flat) % width:
        raise ValueError(f"pointer table rows must have {width} entries")
    return (ctypes.c_uint64 * max(len(flat), 1))(*flat)


def _groups(num_groups, ps, g, tables=()):
    """The group count to pass to C: ``num_groups`` or the rows of the sizes
    table. It may not exceed the rows of any marshalled table, or the library
    would read host memory past the ctypes arrays."""
    if num_groups is None:
        return g
    n = int(num_groups)
    rows = [len(ps) // 4] + [len(t) // w for t, w in tables]
    if n > min(rows):
        raise ValueError(f"num_groups {n} exceeds the rows of the argument tables ({min(rows)})")
    return n


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return ctypes.c_void_p(0)
    if isinstance(stream, ctypes.c_void_p):
        return stream
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def prepare(problem_sizes=None, ptrs_abc=None, ptrs_sfa_sfb=None, stream=None):
    """Marshal arguments once: returns the ctypes arrays (and stream handle) that
    every entry point accepts as they are, for callers that issue the same
    call many times (a timed loop, a captured graph)."""
    out = []
    if problem_sizes is not None:
        out.append(_sizes(problem_sizes)[0])
    if ptrs_abc is not None:
        out.append(_u64(ptrs_abc, 3))
    if ptrs_sfa_sfb is not None:
        out.append(_u64(ptrs_sfa_sfb, 2))
    if stream is not None:
        out.append(_stream(stream))
    return tuple(out)


def nvfp4_grouped_gemm(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None, stream=None) -> None:
    """Enqueue the grouped GEMM; ``problem_sizes`` rows (m, n, k, l), ``ptrs_abc``
    rows (A, B, C) device addresses, ``ptrs_sfa_sfb`` rows (SFA, SFB)."""
    nvfp4_grouped_gemm_config(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups, stream, -1)


def nvfp4_grouped_gemm_config(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None, stream=None,
                              tile_config=-1) -> None:
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    rc = lib.nvfp4_grouped_gemm_config(ps, abc, sf, g, _stream(stream), int(tile_config))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm")


def nvfp4_grouped_gemm_validate(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None) -> int:
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    return lib.nvfp4_grouped_gemm_validate(ps, abc, sf, g)


def nvfp4_num_tile_configs() -> int:
    return load_library().nvfp4_num_tile_configs()


def nvfp4_tile_config_info(cfg: int):
    v = [ctypes.c_int() for _ in range(4)]
    rc = load_library().nvfp4_tile_config_info(int(cfg), *[ctypes.byref(x) for x in v])
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_tile_config_info")
    return dict(bm=v[0].value, bn=v[1].value, bk=v[2].value, threads=v[3].value)


def nvfp4_select_tile_config(problem_sizes, num_cus: int, num_groups=None) -> int:
    ps, g = _sizes(problem_sizes)
    return load_library().nvfp4_select_tile_config(ps, _groups(num_groups, ps, g), int(num_cus))


def nvfp4_launch_geometry(problem_sizes, num_cus: int, cfg: int = -1, split: int = -1, num_groups=None):
    ps, g = _sizes(problem_sizes)
    tiles, grid, used = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int()
    ws = ctypes.c_size_t()
    rc = load_library().nvfp4_launch_geometry(ps, _groups(num_groups, ps, g), int(num_cus),
                                              int(cfg), int(split), ctypes.byref(tiles), ctypes.byref(grid),
                                              ctypes.byref(used), ctypes.byref(ws))
    if rc < 0:
        raise Nvfp4Error(rc, "nvfp4_launch_geometry")
    return dict(config=rc, total_tiles=tiles.value, grid=grid.value, split=used.value, workspace_bytes=ws.value)


def nvfp4_splits_k_over_waves(problem_sizes, num_cus: int, cfg: int = -1, split: int = -1, num_groups=None) -> bool:
    """Whether the plan runs the kernels that split K over the waves in every tile."""
    ps, g = _sizes(problem_sizes)
    rc = load_library().nvfp4_splits_k_over_waves(ps, _groups(num_groups, ps, g), int(num_cus), int(cfg), int(split))
    if rc < 0:
        raise Nvfp4Error(rc, "nvfp4_splits_k_over_waves")
    return rc == 1


def nvfp4_grouped_gemm_ex(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None, workspace=0, workspace_bytes=0,
                          tile_config=-1, split_mode=-1, stream=None) -> None:
    """Grouped GEMM with a caller workspace (device address) and explicit choices."""
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    rc = lib.nvfp4_grouped_gemm_ex(ps, abc, sf, g, ctypes.c_void_p(int(workspace)), int(workspace_bytes),
                                   int(tile_config), int(split_mode), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm_ex")


def nvfp4_grouped_gemm_scratch(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None, tile_config=-1,
                               split_mode=-1, stream=None) -> None:
    """As nvfp4_grouped_gemm_ex with the library's fixed device scratch array
    (NVFP4_SCRATCH_BYTES) as the workspace: allocates nothing. Calls that may
    overlap in time on one device share that array and must not be issued."""
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    rc = lib.nvfp4_grouped_gemm_scratch(ps, abc, sf, g, int(tile_config), int(split_mode), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm_scratch")


def nvfp4_grouped_gemm_stages(problem_sizes, ptrs_abc, ptrs_sfa_sfb, num_groups=None, workspace=0,
                              workspace_bytes=0, tile_config=-1, split_mode=-1, stages=4, stream=None) -> None:
    """As nvfp4_grouped_gemm_ex with the LDS pipeline depth chosen (3 or 4);
    for verification (the results are bitwise those of the default depth)."""
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    rc = lib.nvfp4_grouped_gemm_stages(ps, abc, sf, g, ctypes.c_void_p(int(workspace)), int(workspace_bytes),
                                       int(tile_config), int(split_mode), int(stages), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm_stages")


def nvfp4_grouped_gemm_pow2(problem_sizes, ptrs_abc, ptrs_sfa_sfb, d_status, num_groups=None, workspace=0,
                            workspace_bytes=0, tile_config=-1, split_mode=-1, stream=None) -> None:
    """Grouped GEMM for scales that are all zero or positive powers of two
    (FP4 MFMA with E8M0 scales). ``d_status`` is the device address of an
    int32 the caller clears; the kernel stores 1 there if a scale it used is
    outside that set (then C is not valid)."""
    lib = load_library()
    ps, g = _sizes(problem_sizes)
    abc, sf = _u64(ptrs_abc, 3), _u64(ptrs_sfa_sfb, 2)
    g = _groups(num_groups, ps, g, ((abc, 3), (sf, 2)))
    rc = lib.nvfp4_grouped_gemm_pow2(ps, abc, sf, g, ctypes.c_void_p(int(d_status)),
                                     ctypes.c_void_p(int(workspace)), int(workspace_bytes), int(tile_config),
                                     int(split_mode), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm_pow2")


def nvfp4_grouped_gemm_device(d_problem_sizes, d_ptrs_abc, d_ptrs_sfa_sfb, num_groups, tile_config=-1,
                              d_status=0, stream=None) -> None:
    """Grouped GEMM over group tables in device memory: the first three
    arguments are device addresses of int32 [G][4] (m, n, k, l), uint64 [G][3]
    (A, B, C) and uint64 [G][2] (SFA, SFB); ``d_status`` is the device address
    of an int32 that receives the number of rejected groups (0 = none)."""
    rc = load_library().nvfp4_grouped_gemm_device(
        ctypes.c_void_p(int(d_problem_sizes)), ctypes.c_void_p(int(d_ptrs_abc)), ctypes.c_void_p(int(d_ptrs_sfa_sfb)),
        int(num_groups), int(tile_config), ctypes.c_void_p(int(d_status)), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_grouped_gemm_device")


def nvfp4_device_group_tiles(size, ptrs, tile_config=-1) -> int:
    """Host copy of the device-table kernel's per-group check: tiles of the
    group (m, n, k, l) with addresses (A, B, C, SFA, SFB), or -1 if rejected."""
    sz = (ctypes.c_int32 * 4)(*[int(v) for v in size])
    p = (ctypes.c_uint64 * 5)(*[int(v) for v in ptrs])
    return int(load_library().nvfp4_device_group_tiles(sz, p, int(tile_config)))


def nvfp4_workspace_bytes(problem_sizes, num_cus: int, num_groups=None) -> int:
    ps, g = _sizes(problem_sizes)
    return int(load_library().nvfp4_workspace_bytes(ps, _groups(num_groups, ps, g), int(num_cus)))


def nvfp4_split_plan(problem_sizes, num_cus: int, cfg: int = -1, num_groups=None):
    """How a stream-K call divides the work: (whole_tiles, unit_ranges), the
    tiles dealt out whole first and each workgroup's range of the other
    tiles' (tile, stage) units (unit_ranges[w] .. unit_ranges[w + 1])."""
    ps, g = _sizes(problem_sizes)
    g = _groups(num_groups, ps, g)
    whole = ctypes.c_int32()
    ranges = (ctypes.c_int32 * 1025)()
    rc = load_library().nvfp4_split_plan(ps, g, int(num_cus), int(cfg), ctypes.byref(whole), ranges, 1025)
    if rc < 0:
        raise Nvfp4Error(rc, "nvfp4_split_plan")
    return whole.value, list(ranges[: rc + 1])


def nvfp4_sf_bytes(rows: int, k: int, l: int = 1) -> int:
    return int(load_library().nvfp4_sf_bytes(int(rows), int(k), int(l)))


def nvfp4_last_hip_error() -> int:
    return load_library().nvfp4_last_hip_error()


def nvfp4_error_string(code: int) -> str:
    return load_library().nvfp4_error_string(int(code)).decode()
