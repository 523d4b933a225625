"""ctypes binding of the mainloop measurement kernels (include/nvfp4_mainloop_probe.h,
``libnvfp4_mainloop_probe.so``): the inner loops of the two exact ways of applying
NVFP4's per-16 E4M3 scales on gfx950, and the scaled FP4 conversion's use of its
scale. Argument marshalling only; used by ``bench.py --mainloop-probe`` and the
GPU tests, not by the grouped GEMM."""
from __future__ import annotations

import ctypes
import os

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_mainloop_probe.so")

VARIANT_DEQUANT_F16 = 0   # (b) exact dequantisation to f16, v_mfma_f32_32x32x16_f16
VARIANT_FP4_VALU = 1      # (a) FP4 MFMA per 16-block, scale factors applied on the VALU
VARIANT_BARE_F16 = 2      # the f16 MFMA loop alone
VARIANT_BARE_FP4 = 3      # the scaled FP4 MFMA loop alone, one 16-block per 32-K lane slice
VARIANT_BARE_F16_16X16 = 4  # the f16 MFMA loop alone with the 16x16x32 shape
VARIANT_DEQUANT_128X64 = 5  # (b) on a 128x64 wave tile, one wave per SIMD
VARIANT_DEQUANT_128X64_2W = 6  # the same, two waves per SIMD (512-thread workgroups)
VARIANT_DEQUANT_SHARED_B = 7  # (b) on 64x128 wave tiles with B dequantised once per workgroup, shared in LDS
VARIANT_DEQUANT_SHARED_B_AHEAD = 8  # the same with the exchange a step ahead
VARIANT_BARE_F16_6BIT = 9  # the bare f16 loop on 6-significant-bit operands (like a * s)
VARIANT_BARE_BF16_6BIT = 10  # the bare bf16 loop on 6-significant-bit operands
SINK_PER_WORKGROUP = 512

_lib = None


def load_probe_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is not built: run `python -m moe_matmul_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.nvfp4_probe_mainloop.restype = ctypes.c_int
    lib.nvfp4_probe_mainloop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.nvfp4_probe_flops_per_iteration.restype = ctypes.c_double
    lib.nvfp4_probe_flops_per_iteration.argtypes = [ctypes.c_int]
    lib.nvfp4_probe_cvt_scale.restype = ctypes.c_int
    lib.nvfp4_probe_cvt_scale.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.nvfp4_probe_last_hip_error.restype = ctypes.c_int
    lib.nvfp4_probe_last_hip_error.argtypes = []
    _lib = lib
    return lib


def _check(code, what):
    if code != 0:
        raise RuntimeError(f"{what} failed: {code}"
                           + (f", hip error {load_probe_library().nvfp4_probe_last_hip_error()}" if code == -3 else ""))


def nvfp4_probe_mainloop(variant: int, iters: int, grid: int, sink: int, stream: int = 0) -> None:
    _check(load_probe_library().nvfp4_probe_mainloop(variant, iters, grid, sink, stream), "nvfp4_probe_mainloop")


def nvfp4_probe_flops_per_iteration(variant: int) -> float:
    return load_probe_library().nvfp4_probe_flops_per_iteration(variant)


def nvfp4_probe_cvt_scale(scales: int, n: int, out: int, stream: int = 0) -> None:
    _check(load_probe_library().nvfp4_probe_cvt_scale(scales, n, out, stream), "nvfp4_probe_cvt_scale")
