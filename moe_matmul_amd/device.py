"""Device-memory plumbing (PyTorch) for the grouped GEMM: upload seeded byte
arrays, build the host pointer tables and call the library. No arithmetic."""
from __future__ import annotations

import numpy as np
import torch

from ._binding import (nvfp4_grouped_gemm_config, nvfp4_grouped_gemm_device, nvfp4_grouped_gemm_ex,
                       nvfp4_grouped_gemm_pow2)

FP16_NAN_BITS = 0xFFFF


def upload(shapes, groups, device="cuda", c_fill_bits=FP16_NAN_BITS, c_guard=0):
    """Copy each group's bytes to ``device``; allocate C (pre-filled with
    ``c_fill_bits``), optionally inside a guard band of ``c_guard`` fp16 elements
    on each side (kept for canary checks)."""
    if c_guard % 8:
        raise ValueError("c_guard must be a multiple of 8 elements (C stays 16-byte aligned)")
    out = []
    for (m, n, k, l), g in zip(shapes, groups):
        d = {}
        for key in ("a", "b", "sfa", "sfb"):
            arr = np.ascontiguousarray(g[key]).reshape(-1)
            t = torch.empty(max(arr.size, 16), dtype=torch.uint8, device=device)
            if arr.size:
                t[: arr.size].copy_(torch.from_numpy(arr))
            d[key] = t
        numel = l * m * n
        fill = int(np.array(c_fill_bits, dtype=np.uint16).view(np.int16))
        store = torch.full((numel + 2 * c_guard + 8,), fill, dtype=torch.int16, device=device)
        d["c_store"] = store
        d["c"] = store[c_guard: c_guard + numel]
        d["c_guard"] = c_guard
        out.append(d)
    return out


def pointer_tables(dev_groups):
    abc = [(d["a"].data_ptr(), d["b"].data_ptr(), d["c"].data_ptr()) for d in dev_groups]
    sf = [(d["sfa"].data_ptr(), d["sfb"].data_ptr()) for d in dev_groups]
    return abc, sf


def run(shapes, dev_groups, stream=None, tile_config=-1, split_mode=None, workspace=None):
    """Enqueue one grouped GEMM on ``stream`` (default: torch's current stream).

    With ``split_mode`` or ``workspace`` given, the call goes through
    nvfp4_grouped_gemm_ex with that (uint8 tensor) workspace; otherwise through
    nvfp4_grouped_gemm_config (no workspace: whole tiles)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    abc, sf = pointer_tables(dev_groups)
    if split_mode is None and workspace is None:
        nvfp4_grouped_gemm_config(shapes, abc, sf, len(shapes), stream, tile_config)
    else:
        ws_ptr = 0 if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else workspace.numel()
        nvfp4_grouped_gemm_ex(shapes, abc, sf, len(shapes), ws_ptr, ws_bytes, tile_config,
                              -1 if split_mode is None else split_mode, stream)


def run_pow2(shapes, dev_groups, status, stream=None, tile_config=-1, split_mode=-1, workspace=None):
    """Enqueue nvfp4_grouped_gemm_pow2 (scales all zero or powers of two);
    ``status`` is an int32 device tensor the caller has cleared, ``workspace``
    a uint8 device tensor or None (then whole tiles)."""
    if stream is None:
        stream = torch.cuda.current_stream()
    abc, sf = pointer_tables(dev_groups)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel()
    nvfp4_grouped_gemm_pow2(shapes, abc, sf, status.data_ptr(), len(shapes), ws_ptr, ws_bytes, tile_config,
                            split_mode, stream)


def device_tables(shapes, dev_groups, device="cuda"):
    """The group tables of nvfp4_grouped_gemm_device as device tensors:
    int32 [G][4] sizes, int64 [G][3] (A, B, C) and [G][2] (SFA, SFB) addresses."""
    abc, sf = pointer_tables(dev_groups)
    sizes = torch.tensor([list(s) for s in shapes], dtype=torch.int32).reshape(-1, 4)
    as_i64 = lambda rows, w: torch.tensor(np.array(rows, dtype=np.uint64).reshape(-1, w).view(np.int64))
    return sizes.to(device), as_i64(abc, 3).to(device), as_i64(sf, 2).to(device)


def run_device(tables, num_groups, tile_config=-1, status=None, stream=None):
    """Enqueue nvfp4_grouped_gemm_device over ``tables`` (see device_tables);
    ``status`` is an int32 device tensor or None."""
    if stream is None:
        stream = torch.cuda.current_stream()
    sizes, abc, sf = tables
    nvfp4_grouped_gemm_device(sizes.data_ptr(), abc.data_ptr(), sf.data_ptr(), num_groups, tile_config,
                              0 if status is None else status.data_ptr(), stream)


def workspace_for(shapes, device="cuda"):
    """A uint8 workspace tensor large enough for any plan on this device."""
    from ._binding import nvfp4_workspace_bytes
    cus = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
    n = max(nvfp4_workspace_bytes(shapes, cus), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def c_as_numpy(shapes, dev_groups):
    """Copy every C back as numpy float16 [l][m][n]."""
    res = []
    for (m, n, k, l), d in zip(shapes, dev_groups):
        bits = d["c"].cpu().numpy().view(np.uint16)
        res.append(bits.view(np.float16).reshape(l, m, n))
    return res


def guards_intact(dev_groups, c_fill_bits=FP16_NAN_BITS):
    """True when the guard bands around every C still hold the fill pattern."""
    for d in dev_groups:
        g = d["c_guard"]
        if g == 0:
            continue
        st = d["c_store"].cpu().numpy().view(np.uint16)
        n = d["c"].numel()
        if not (np.all(st[:g] == c_fill_bits) and np.all(st[g + n:] == c_fill_bits)):
            return False
    return True
