"""Block-scaled FP8 GEMM (dense, MoE contiguous, MoE masked) for AMD MI355X.

Thin Python binding of ``libfp8bs.so`` (C ABI declared in ``include/fp8bs.h``):
argument checks and marshalling only -- every step of the computation runs in
the library's HIP kernels.  PyTorch supplies device memory (the split-K
workspace included) and the stream.

``fp8bs_*_nt`` map one to one onto the C calls without workspace, and
``fp8bs_*_nt_ws`` onto the workspace calls (a workspace tensor of
``workspace_size(...)`` bytes is allocated on the call's stream when none is
given).  ``dense_nt``, ``grouped_contiguous_nt`` and ``grouped_masked_nt`` are
the workspace variants.

The binding refuses to run without the compiled library; there is no fallback.
Build it with ``python -m moe_grouped_gemm_block_amd.build``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

__all__ = [
    "fp8bs_dense_nt", "fp8bs_grouped_contiguous_nt", "fp8bs_grouped_masked_nt",
    "fp8bs_dense_nt_ws", "fp8bs_grouped_contiguous_nt_ws", "fp8bs_grouped_masked_nt_ws",
    "fp8bs_dense_nt_noalloc", "noalloc_scratch_bytes", "dense_nt", "grouped_contiguous_nt", "grouped_masked_nt",
    "get_mk_alignment", "get_sfa_ld", "set_num_cus", "get_num_cus", "plan_query",
    "workspace_size", "describe_config", "count_tiles", "instances", "force_instance",
    "force_splits", "status_string", "sfa_mn_major", "library_path", "FP8BSError",
    "fp8bs_quantize_1x128", "fp8bs_quantize_128x128", "quantize_1x128", "quantize_128x128",
    "fp8bs_dense_nt_ue8m0", "fp8bs_grouped_contiguous_nt_ue8m0", "fp8bs_grouped_masked_nt_ue8m0",
    "ue8m0_exponents", "pack_ue8m0", "sfa_ue8m0_mn_major", "sfb_ue8m0",
    "fp8bs_dense_nt_c", "fp8bs_grouped_contiguous_nt_c", "fp8bs_grouped_masked_nt_c",
    "fp8bs_dense_nn", "fp8bs_dense_tn", "fp8bs_dense_tt", "fp8bs_k_grouped_tn_contiguous",
    "fp8bs_dense_nn_ue8m0", "fp8bs_dense_tn_ue8m0", "fp8bs_dense_tt_ue8m0",
    "fp8bs_k_grouped_tn_contiguous_ue8m0",
    "LAYOUT_DENSE", "LAYOUT_CONTIGUOUS", "LAYOUT_MASKED", "LAYOUT_K_GROUPED",
    "LAYOUT_DENSE_NN", "LAYOUT_DENSE_TN", "LAYOUT_DENSE_TT", "LAYOUT_UE8M0",
]

LAYOUT_DENSE, LAYOUT_CONTIGUOUS, LAYOUT_MASKED = 0, 1, 2
LAYOUT_K_GROUPED, LAYOUT_DENSE_NN, LAYOUT_DENSE_TN, LAYOUT_DENSE_TT = 3, 4, 5, 6
LAYOUT_UE8M0 = 16                 # OR-ed into a layout code: the packed power-of-two calls

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libfp8bs.so")
_lib = None


class FP8BSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Plan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("waves_m", ctypes.c_int),
                ("waves_n", ctypes.c_int), ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("wg_per_cu", ctypes.c_int), ("stages", ctypes.c_int), ("tiles", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("raster", ctypes.c_int), ("instance", ctypes.c_int),
                ("splits", ctypes.c_int), ("workspace_bytes", ctypes.c_int64),
                ("kind", ctypes.c_int), ("ue8m0", ctypes.c_int), ("mn", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing; build it with "
                           "`python -m moe_grouped_gemm_block_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.fp8bs_dense_nt.argtypes = [P, P, P, P, P, I, I, I, P]
    lib.fp8bs_grouped_contiguous_nt.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    lib.fp8bs_grouped_masked_nt.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
    S = ctypes.c_size_t
    lib.fp8bs_dense_nt_ws.argtypes = [P, P, P, P, P, I, I, I, P, S, P]
    lib.fp8bs_dense_nt_noalloc.argtypes = [P, P, P, P, P, I, I, I, P]
    lib.fp8bs_dense_nt_noalloc.restype = I
    lib.fp8bs_noalloc_scratch_bytes.restype = S
    lib.fp8bs_grouped_contiguous_nt_ws.argtypes = [P, P, P, P, P, P, I, I, I, I, P, S, P]
    lib.fp8bs_grouped_masked_nt_ws.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, S, P]
    for f in ("fp8bs_dense_nt", "fp8bs_grouped_contiguous_nt", "fp8bs_grouped_masked_nt",
              "fp8bs_dense_nt_ws", "fp8bs_grouped_contiguous_nt_ws", "fp8bs_grouped_masked_nt_ws",
              "fp8bs_get_mk_alignment", "fp8bs_set_num_cus", "fp8bs_get_num_cus",
              "fp8bs_plan_query", "fp8bs_describe_config"):
        getattr(lib, f).restype = I
    lib.fp8bs_get_sfa_ld.argtypes = [I64]
    lib.fp8bs_get_sfa_ld.restype = I64
    lib.fp8bs_set_num_cus.argtypes = [I]
    lib.fp8bs_plan_query.argtypes = [I, I64, I, I, I, I, I, I64, ctypes.POINTER(_Plan)]
    lib.fp8bs_workspace_size.argtypes = [I, I64, I, I, I, I]
    lib.fp8bs_workspace_size.restype = I64
    lib.fp8bs_force_splits.argtypes = [I]
    lib.fp8bs_force_splits.restype = I
    lib.fp8bs_dense_nt_c.argtypes = [P, P, P, P, P, P, I, I, I, P, S, P]
    lib.fp8bs_grouped_contiguous_nt_c.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, S, P]
    lib.fp8bs_grouped_masked_nt_c.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, S, P]
    for f in ("fp8bs_dense_nt_c", "fp8bs_grouped_contiguous_nt_c", "fp8bs_grouped_masked_nt_c"):
        getattr(lib, f).restype = I
    lib.fp8bs_dense_nt_ue8m0.argtypes = [P, P, P, P, P, I, I, I, P, S, P]
    lib.fp8bs_grouped_contiguous_nt_ue8m0.argtypes = [P, P, P, P, P, P, I, I, I, I, P, S, P]
    lib.fp8bs_grouped_masked_nt_ue8m0.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, S, P]
    for f in ("fp8bs_dense_nt_ue8m0", "fp8bs_grouped_contiguous_nt_ue8m0",
              "fp8bs_grouped_masked_nt_ue8m0"):
        getattr(lib, f).restype = I
    lib.fp8bs_quantize_1x128.argtypes = [P, I, P, P, I, I, I, P]
    lib.fp8bs_quantize_1x128.restype = I
    lib.fp8bs_quantize_128x128.argtypes = [P, I, P, P, I, I, I, P]
    lib.fp8bs_quantize_128x128.restype = I
    for f in ("nn", "tn", "tt"):
        getattr(lib, "fp8bs_dense_" + f).argtypes = [P, P, P, P, P, P, I, I, I, P, S, P]
    lib.fp8bs_k_grouped_tn_contiguous.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, S, P]
    for f in ("nn", "tn", "tt"):
        getattr(lib, "fp8bs_dense_" + f + "_ue8m0").argtypes = [P, P, P, P, P, P, I, I, I, P, S, P]
    lib.fp8bs_k_grouped_tn_contiguous_ue8m0.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, S, P]
    lib.fp8bs_describe_config.argtypes = [I, I64, I, I, I, I, ctypes.c_char_p, ctypes.c_size_t]
    lib.fp8bs_count_tiles.argtypes = [I, I64, I, I, I, I]
    lib.fp8bs_count_tiles.restype = I64
    lib.fp8bs_num_instances.restype = I
    lib.fp8bs_force_instance.argtypes = [I]
    lib.fp8bs_force_instance.restype = I
    lib.fp8bs_instance_info.argtypes = [I, ctypes.POINTER(_Plan)]
    lib.fp8bs_instance_info.restype = I
    lib.fp8bs_status_string.argtypes = [I]
    lib.fp8bs_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return _load().fp8bs_status_string(int(status)).decode()


def get_mk_alignment() -> int:
    return int(_load().fp8bs_get_mk_alignment())


def get_sfa_ld(rows: int) -> int:
    return int(_load().fp8bs_get_sfa_ld(int(rows)))


def set_num_cus(n: int) -> int:
    return int(_load().fp8bs_set_num_cus(int(n)))


def get_num_cus() -> int:
    return int(_load().fp8bs_get_num_cus())


def plan_query(layout: int, m: int, n: int, k: int, num_groups: int = 1, expected_m: int = 0,
               num_cus: int = 256, workspace_bytes: int = 0) -> dict:
    plan = _Plan()
    st = _load().fp8bs_plan_query(int(layout), int(m), int(n), int(k), int(num_groups),
                                  int(expected_m), int(num_cus), int(workspace_bytes),
                                  ctypes.byref(plan))
    if st != 0:
        raise FP8BSError(st, "fp8bs_plan_query")
    return {name: getattr(plan, name) for name, _ in _Plan._fields_}


def workspace_size(layout: int, m: int, n: int, k: int, num_groups: int = 1,
                   expected_m: int = 0) -> int:
    """Workspace bytes the preferred plan uses on the current device (0: no split)."""
    v = int(_load().fp8bs_workspace_size(int(layout), int(m), int(n), int(k), int(num_groups),
                                         int(expected_m)))
    if v < 0:
        raise FP8BSError(-v, "fp8bs_workspace_size")
    return v


def count_tiles(layout: int, m: int, n: int, num_groups: int, block_m: int, block_n: int) -> int:
    return int(_load().fp8bs_count_tiles(int(layout), int(m), int(n), int(num_groups),
                                         int(block_m), int(block_n)))


def instances() -> list:
    lib = _load()
    out = []
    for i in range(lib.fp8bs_num_instances()):
        plan = _Plan()
        _check(lib.fp8bs_instance_info(i, ctypes.byref(plan)), "fp8bs_instance_info")
        out.append({name: getattr(plan, name) for name, _ in _Plan._fields_})
    return out


def force_instance(i: int) -> int:
    """Pin every later call of this thread to compiled instance i (-1 = planner's choice);
    returns the previous."""
    prev = int(_load().fp8bs_force_instance(int(i)))
    if prev == -2:
        raise ValueError(f"no compiled instance {i}")
    return prev


def force_splits(s: int) -> int:
    """Pin the K split count of this thread's later workspace calls (0 = planner's choice);
    returns the previous."""
    prev = int(_load().fp8bs_force_splits(int(s)))
    if prev == -1:
        raise ValueError(f"invalid split count {s}")
    return prev


def describe_config(layout: int, m: int, n: int, k: int, num_groups: int = 1,
                    expected_m: int = 0) -> str:
    buf = ctypes.create_string_buffer(512)
    st = _load().fp8bs_describe_config(int(layout), int(m), int(n), int(k), int(num_groups),
                                       int(expected_m), buf, 512)
    if st != 0:
        raise FP8BSError(st, "fp8bs_describe_config")
    return buf.value.decode()


# ---- tensor marshalling ----------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes, ndim=None):
    torch = _torch()
    # common case first: a contiguous device tensor of an accepted dtype
    if (type(t) is torch.Tensor and t.is_cuda and t.dtype in dtypes and t.is_contiguous()
            and (ndim is None or t.dim() == ndim)):
        return ctypes.c_void_p(t.data_ptr())
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


_DTYPES = {}


def _fp8_dtypes():
    d = _DTYPES.get("fp8")
    if d is None:
        torch = _torch()
        d = _DTYPES["fp8"] = (torch.uint8, torch.float8_e4m3fn)
    return d


def _bf16_dtypes():
    d = _DTYPES.get("bf16")
    if d is None:
        torch = _torch()
        d = _DTYPES["bf16"] = (torch.bfloat16, torch.int16, torch.uint16)
    return d


_NO_SWITCH = contextlib.nullcontext()


def _on_device(t):
    """Context that makes t's device current (nothing to do when it already is)."""
    torch = _torch()
    idx = t.get_device()
    if idx == torch.cuda.current_device():
        return _NO_SWITCH
    return torch.cuda.device(idx)


def _stream_handle(stream, device):
    """Raw HIP stream handle: the given torch stream, or the device's current stream."""
    torch = _torch()
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(device.index if device.index is not None
                                       else torch.cuda.current_device()))
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def sfa_mn_major(sa, rows_ld: Optional[int] = None):
    """Logical A scales [..., rows, K/128] -> MN-major storage [..., K/128, ld(rows)].

    Works on torch tensors (any device) and returns a contiguous tensor whose
    padding columns are zero.  Layout helper, analogous to the pages'
    transform_sf_into_required_layout."""
    torch = _torch()
    rows, kb = sa.shape[-2], sa.shape[-1]
    ld = get_sfa_ld(rows) if rows_ld is None else rows_ld
    out = torch.zeros(*sa.shape[:-2], kb, ld, dtype=torch.float32, device=sa.device)
    out[..., :, :rows] = sa.transpose(-1, -2)
    return out


def _check(st: int, where: str):
    if st != 0:
        raise FP8BSError(st, where)


def _workspace(ws, layout, m, n, k, g, expected_m, stream, device):
    """(pointer, bytes, tensor) of the workspace for a _ws call: the caller's uint8 device
    tensor, or a fresh one of workspace_size() bytes allocated on the call's stream."""
    torch = _torch()
    if ws is None:
        nbytes = workspace_size(layout, m, n, k, g, expected_m)
        if nbytes == 0:
            return ctypes.c_void_p(None), 0, None
        with torch.cuda.stream(_stream(stream, device)):
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ptr = _dev_ptr(ws, "workspace", (torch.uint8,), 1)
    return ptr, ws.numel(), ws


def _dense_args(a, sfa, b, sfb, d):
    torch = _torch()
    m, k = a.shape
    n = b.shape[0]
    kb = k // 128 if k % 128 == 0 else -1
    args = (_dev_ptr(a, "a", _fp8_dtypes(), 2), _dev_ptr(sfa, "sfa", (torch.float32,)),
            _dev_ptr(b, "b", _fp8_dtypes(), 2), _dev_ptr(sfb, "sfb", (torch.float32,)),
            _dev_ptr(d, "d", _bf16_dtypes(), 2))
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if kb > 0 and (sfa.numel() != kb * get_sfa_ld(m) or sfb.numel() != ((n + 127) // 128) * kb):
        raise ValueError("scale tensor sizes do not match the shapes")
    return args, m, n, k


def _contiguous_args(a, sfa, b, sfb, d, grouped_layout):
    torch = _torch()
    m, k = a.shape
    g, n = b.shape[0], b.shape[1]
    kb = k // 128 if k % 128 == 0 else -1
    args = (_dev_ptr(a, "a", _fp8_dtypes(), 2), _dev_ptr(sfa, "sfa", (torch.float32,)),
            _dev_ptr(b, "b", _fp8_dtypes(), 3), _dev_ptr(sfb, "sfb", (torch.float32,)),
            _dev_ptr(d, "d", _bf16_dtypes(), 2),
            _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), 1))
    if b.shape[2] != k or tuple(d.shape) != (m, n) or grouped_layout.shape[0] != m:
        raise ValueError("shape mismatch between a, b, d and grouped_layout")
    if kb > 0 and (sfa.numel() != kb * get_sfa_ld(m) or sfb.numel() != g * ((n + 127) // 128) * kb):
        raise ValueError("scale tensor sizes do not match the shapes")
    return args, m, n, k, g


def _masked_args(a, sfa, b, sfb, d, masked_m):
    torch = _torch()
    g, max_m, k = a.shape
    n = b.shape[1]
    kb = k // 128 if k % 128 == 0 else -1
    args = (_dev_ptr(a, "a", _fp8_dtypes(), 3), _dev_ptr(sfa, "sfa", (torch.float32,)),
            _dev_ptr(b, "b", _fp8_dtypes(), 3), _dev_ptr(sfb, "sfb", (torch.float32,)),
            _dev_ptr(d, "d", _bf16_dtypes(), 3), _dev_ptr(masked_m, "masked_m", (torch.int32,), 1))
    if b.shape[0] != g or b.shape[2] != k or tuple(d.shape) != (g, max_m, n) or masked_m.shape[0] != g:
        raise ValueError("shape mismatch between a, b, d and masked_m")
    if kb > 0 and (sfa.numel() != g * kb * get_sfa_ld(max_m)
                   or sfb.numel() != g * ((n + 127) // 128) * kb):
        raise ValueError("scale tensor sizes do not match the shapes")
    return args, g, max_m, n, k


def _stream(stream, device):
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def fp8bs_dense_nt(a, sfa, b, sfb, d, stream=None):
    """D[m][n] = A[m][k] * B[n][k]^T with 1x128 A scales and 128x128 B scales.

    a: e4m3 [m][k]; sfa: f32 MN-major [k/128][ld(m)]; b: e4m3 [n][k];
    sfb: f32 [ceil(n/128)][k/128]; d: bf16 [m][n] (written)."""
    args, m, n, k = _dense_args(a, sfa, b, sfb, d)
    with _on_device(a):
        st = _load().fp8bs_dense_nt(*args, m, n, k, _stream_handle(stream, a.device))
    _check(st, "fp8bs_dense_nt")


def fp8bs_dense_nt_ws(a, sfa, b, sfb, d, workspace=None, stream=None):
    """fp8bs_dense_nt with a split-K workspace (uint8 device tensor, or None to allocate)."""
    args, m, n, k = _dense_args(a, sfa, b, sfb, d)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_DENSE, m, n, k, 1, 0, s, a.device)
        st = _load().fp8bs_dense_nt_ws(*args, m, n, k, wp, wb, _stream_handle(s, a.device))
    _check(st, "fp8bs_dense_nt_ws")


def fp8bs_dense_nt_noalloc(a, sfa, b, sfb, d, stream=None):
    """fp8bs_dense_nt_ws with the split-K workspace taken from the library's own per-device
    scratch array (nothing is allocated); calls that overlap on one GPU race on it."""
    args, m, n, k = _dense_args(a, sfa, b, sfb, d)
    with _on_device(a):
        st = _load().fp8bs_dense_nt_noalloc(*args, m, n, k, _stream_handle(stream, a.device))
    _check(st, "fp8bs_dense_nt_noalloc")


def noalloc_scratch_bytes() -> int:
    return int(_load().fp8bs_noalloc_scratch_bytes())


def fp8bs_grouped_contiguous_nt(a, sfa, b, sfb, d, grouped_layout, stream=None):
    """Contiguous MoE layout: a [m_total][k], b [g][n][k], grouped_layout int32 [m_total]."""
    args, m, n, k, g = _contiguous_args(a, sfa, b, sfb, d, grouped_layout)
    with _on_device(a):
        st = _load().fp8bs_grouped_contiguous_nt(*args, m, n, k, g, _stream_handle(stream, a.device))
    _check(st, "fp8bs_grouped_contiguous_nt")


def fp8bs_grouped_contiguous_nt_ws(a, sfa, b, sfb, d, grouped_layout, workspace=None, stream=None):
    """fp8bs_grouped_contiguous_nt with a split-K workspace."""
    args, m, n, k, g = _contiguous_args(a, sfa, b, sfb, d, grouped_layout)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_CONTIGUOUS, m, n, k, g, 0, s, a.device)
        st = _load().fp8bs_grouped_contiguous_nt_ws(*args, m, n, k, g, wp, wb,
                                                    _stream_handle(s, a.device))
    _check(st, "fp8bs_grouped_contiguous_nt_ws")


def fp8bs_grouped_masked_nt(a, sfa, b, sfb, d, masked_m, expected_m: int = 0, stream=None):
    """Masked MoE layout: a [g][max_m][k], b [g][n][k], d [g][max_m][n], masked_m int32 [g]."""
    args, g, max_m, n, k = _masked_args(a, sfa, b, sfb, d, masked_m)
    with _on_device(a):
        st = _load().fp8bs_grouped_masked_nt(*args, g, max_m, int(expected_m), n, k,
                                             _stream_handle(stream, a.device))
    _check(st, "fp8bs_grouped_masked_nt")


def fp8bs_grouped_masked_nt_ws(a, sfa, b, sfb, d, masked_m, expected_m: int = 0, workspace=None,
                               stream=None):
    """fp8bs_grouped_masked_nt with a split-K workspace."""
    args, g, max_m, n, k = _masked_args(a, sfa, b, sfb, d, masked_m)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_MASKED, max_m, n, k, g, int(expected_m), s,
                                   a.device)
        st = _load().fp8bs_grouped_masked_nt_ws(*args, g, max_m, int(expected_m), n, k, wp, wb,
                                                _stream_handle(s, a.device))
    _check(st, "fp8bs_grouped_masked_nt_ws")


dense_nt = fp8bs_dense_nt_ws
grouped_contiguous_nt = fp8bs_grouped_contiguous_nt_ws
grouped_masked_nt = fp8bs_grouped_masked_nt_ws


# ---- quantisers ------------------------------------------------------------

DTYPE_F32, DTYPE_BF16 = 0, 1


def _x_dtype(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return DTYPE_F32
    if x.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"quantiser input must be float32 or bfloat16, got {x.dtype}")


def fp8bs_quantize_1x128(x, q, sfa, stream=None):
    """Activations x f32/bf16 [rows][k] or [G][rows][k] -> q e4m3 (same shape) and sfa
    f32 MN-major [(G,) k/128, ld(rows)] (the GEMM's A-scale layout)."""
    torch = _torch()
    if x.dim() not in (2, 3):
        raise ValueError("x must be [rows][k] or [G][rows][k]")
    G = 1 if x.dim() == 2 else x.shape[0]
    rows, k = x.shape[-2], x.shape[-1]
    xp = _dev_ptr(x, "x", (torch.float32, torch.bfloat16))
    qp = _dev_ptr(q, "q", _fp8_dtypes())
    sp = _dev_ptr(sfa, "sfa", (torch.float32,))
    if tuple(q.shape) != tuple(x.shape):
        raise ValueError("q must have x's shape")
    if k % 128 == 0 and sfa.numel() != G * (k // 128) * get_sfa_ld(rows):
        raise ValueError("sfa must hold [G][k/128][ld(rows)] floats")
    with _on_device(x):
        st = _load().fp8bs_quantize_1x128(xp, _x_dtype(x), qp, sp, G, rows, k,
                                          _stream_handle(stream, x.device))
    _check(st, "fp8bs_quantize_1x128")


def fp8bs_quantize_128x128(x, q, sfb, stream=None):
    """Weights x f32/bf16 [n][k] or [G][n][k] -> q e4m3 (same shape), sfb f32
    [(G,) ceil(n/128), k/128]."""
    torch = _torch()
    if x.dim() not in (2, 3):
        raise ValueError("x must be [n][k] or [G][n][k]")
    G = 1 if x.dim() == 2 else x.shape[0]
    n, k = x.shape[-2], x.shape[-1]
    xp = _dev_ptr(x, "x", (torch.float32, torch.bfloat16))
    qp = _dev_ptr(q, "q", _fp8_dtypes())
    sp = _dev_ptr(sfb, "sfb", (torch.float32,))
    if tuple(q.shape) != tuple(x.shape):
        raise ValueError("q must have x's shape")
    if k % 128 == 0 and sfb.numel() != G * ((n + 127) // 128) * (k // 128):
        raise ValueError("sfb must hold [G][ceil(n/128)][k/128] floats")
    with _on_device(x):
        st = _load().fp8bs_quantize_128x128(xp, _x_dtype(x), qp, sp, G, n, k,
                                            _stream_handle(stream, x.device))
    _check(st, "fp8bs_quantize_128x128")


def quantize_1x128(x, stream=None):
    """Allocating form: returns (q uint8, sfa f32 MN-major)."""
    torch = _torch()
    G = 1 if x.dim() == 2 else x.shape[0]
    rows, k = x.shape[-2], x.shape[-1]
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    shape = (k // 128, get_sfa_ld(rows)) if x.dim() == 2 else (G, k // 128, get_sfa_ld(rows))
    sfa = torch.zeros(shape, dtype=torch.float32, device=x.device)
    fp8bs_quantize_1x128(x, q, sfa, stream)
    return q, sfa


def quantize_128x128(x, stream=None):
    """Allocating form: returns (q uint8, sfb f32)."""
    torch = _torch()
    n, k = x.shape[-2], x.shape[-1]
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    shape = ((n + 127) // 128, k // 128) if x.dim() == 2 else (x.shape[0], (n + 127) // 128, k // 128)
    sfb = torch.empty(shape, dtype=torch.float32, device=x.device)
    fp8bs_quantize_128x128(x, q, sfb, stream)
    return q, sfb


# ---- power-of-two (packed UE8M0) scales -------------------------------------

def ue8m0_exponents(s):
    """Powers of two (float32 tensor) -> their biased E8M0 exponents e (s = 2^(e-127)),
    int32.  Raises if a value is not a power of two in [2^-127, 2^127]."""
    torch = _torch()
    m, e = torch.frexp(s.float())
    if not bool(torch.all(m == 0.5)):
        raise ValueError("UE8M0 scales must be powers of two")
    out = (e - 1 + 127).to(torch.int32)
    if bool(torch.any(out < 0)) or bool(torch.any(out > 254)):
        raise ValueError("UE8M0 exponent out of range")
    return out


def pack_ue8m0(e):
    """Exponents [..., groups] -> int32 [..., ceil(groups/4)], byte j of word w = group 4w+j."""
    torch = _torch()
    kb = e.shape[-1]
    w = (kb + 3) // 4
    pad = torch.zeros(*e.shape[:-1], 4 * w, dtype=torch.int64, device=e.device)
    pad[..., :kb] = e.to(torch.int64) & 0xFF
    pad = pad.reshape(*e.shape[:-1], w, 4)
    v = pad[..., 0] | (pad[..., 1] << 8) | (pad[..., 2] << 16) | (pad[..., 3] << 24)
    v = torch.where(v >= 2 ** 31, v - 2 ** 32, v)
    return v.to(torch.int32)


def sfa_ue8m0_mn_major(sa):
    """Power-of-two A scales [..., rows, K/128] -> packed int32 MN-major
    [..., ceil(K/512), ld(rows)] (padding zero)."""
    torch = _torch()
    rows = sa.shape[-2]
    packed = pack_ue8m0(ue8m0_exponents(sa))                 # [..., rows, w]
    ld = get_sfa_ld(rows)
    out = torch.zeros(*packed.shape[:-2], packed.shape[-1], ld, dtype=torch.int32,
                      device=sa.device)
    out[..., :, :rows] = packed.transpose(-1, -2)
    return out.contiguous()


def sfb_ue8m0(sb):
    """Power-of-two B scales [..., ceil(N/128), K/128] -> packed int32
    [..., ceil(N/128), ceil(K/512)]."""
    return pack_ue8m0(ue8m0_exponents(sb)).contiguous()


def _ue8m0_checks(sfa, sfb, a_slots, b_groups, rows, n, k):
    torch = _torch()
    w = (k // 128 + 3) // 4 if k % 128 == 0 else -1
    if w > 0 and (sfa.numel() != a_slots * w * get_sfa_ld(rows)
                  or sfb.numel() != b_groups * ((n + 127) // 128) * w):
        raise ValueError("packed UE8M0 scale tensor sizes do not match the shapes")
    return (_dev_ptr(sfa, "sfa", (torch.int32,)), _dev_ptr(sfb, "sfb", (torch.int32,)))


def _opt_workspace(ws):
    torch = _torch()
    if ws is None:
        return ctypes.c_void_p(None), 0
    return _dev_ptr(ws, "workspace", (torch.uint8,), 1), ws.numel()


def fp8bs_dense_nt_ue8m0(a, sfa, b, sfb, d, workspace=None, stream=None):
    """Dense GEMM with packed UE8M0 scales (sfa int32 MN-major [ceil(k/512)][ld(m)],
    sfb int32 [ceil(n/128)][ceil(k/512)]); workspace (uint8) optional, enables split-K."""
    torch = _torch()
    m, k = a.shape
    n = b.shape[0]
    ap = _dev_ptr(a, "a", _fp8_dtypes(), 2)
    bp = _dev_ptr(b, "b", _fp8_dtypes(), 2)
    dp = _dev_ptr(d, "d", _bf16_dtypes(), 2)
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    sap, sbp = _ue8m0_checks(sfa, sfb, 1, 1, m, n, k)
    wp, wb = _opt_workspace(workspace)
    with _on_device(a):
        st = _load().fp8bs_dense_nt_ue8m0(ap, sap, bp, sbp, dp, m, n, k, wp, wb,
                                          _stream_handle(stream, a.device))
    _check(st, "fp8bs_dense_nt_ue8m0")


def fp8bs_grouped_contiguous_nt_ue8m0(a, sfa, b, sfb, d, grouped_layout, workspace=None,
                                      stream=None):
    """Contiguous MoE layout with packed UE8M0 scales (sfb [g][ceil(n/128)][ceil(k/512)])."""
    torch = _torch()
    m, k = a.shape
    g, n = b.shape[0], b.shape[1]
    ap = _dev_ptr(a, "a", _fp8_dtypes(), 2)
    bp = _dev_ptr(b, "b", _fp8_dtypes(), 3)
    dp = _dev_ptr(d, "d", _bf16_dtypes(), 2)
    lp = _dev_ptr(grouped_layout, "grouped_layout", (torch.int32,), 1)
    if b.shape[2] != k or tuple(d.shape) != (m, n) or grouped_layout.shape[0] != m:
        raise ValueError("shape mismatch between a, b, d and grouped_layout")
    sap, sbp = _ue8m0_checks(sfa, sfb, 1, g, m, n, k)
    wp, wb = _opt_workspace(workspace)
    with _on_device(a):
        st = _load().fp8bs_grouped_contiguous_nt_ue8m0(ap, sap, bp, sbp, dp, lp, m, n, k, g, wp,
                                                       wb, _stream_handle(stream, a.device))
    _check(st, "fp8bs_grouped_contiguous_nt_ue8m0")


def fp8bs_grouped_masked_nt_ue8m0(a, sfa, b, sfb, d, masked_m, expected_m: int = 0,
                                  workspace=None, stream=None):
    """Masked MoE layout with packed UE8M0 scales (sfa [g][ceil(k/512)][ld(max_m)])."""
    torch = _torch()
    g, max_m, k = a.shape
    n = b.shape[1]
    ap = _dev_ptr(a, "a", _fp8_dtypes(), 3)
    bp = _dev_ptr(b, "b", _fp8_dtypes(), 3)
    dp = _dev_ptr(d, "d", _bf16_dtypes(), 3)
    mp = _dev_ptr(masked_m, "masked_m", (torch.int32,), 1)
    if b.shape[0] != g or b.shape[2] != k or tuple(d.shape) != (g, max_m, n):
        raise ValueError("shape mismatch between a, b, d and masked_m")
    sap, sbp = _ue8m0_checks(sfa, sfb, g, g, max_m, n, k)
    wp, wb = _opt_workspace(workspace)
    with _on_device(a):
        st = _load().fp8bs_grouped_masked_nt_ue8m0(ap, sap, bp, sbp, dp, mp, g, max_m,
                                                   int(expected_m), n, k, wp, wb,
                                                   _stream_handle(stream, a.device))
    _check(st, "fp8bs_grouped_masked_nt_ue8m0")


# ---- D = C + A B^T ---------------------------------------------------------

def _addend(c, d):
    torch = _torch()
    if tuple(c.shape) != tuple(d.shape):
        raise ValueError("c must have d's shape")
    return _dev_ptr(c, "c", (torch.float32,))


def fp8bs_dense_nt_c(a, sfa, b, sfb, c, d, workspace=None, stream=None):
    """D = bf16(C + A B^T): fp8bs_dense_nt_ws with an FP32 addend c [m][n]."""
    args, m, n, k = _dense_args(a, sfa, b, sfb, d)
    cp = _addend(c, d)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_DENSE, m, n, k, 1, 0, s, a.device)
        st = _load().fp8bs_dense_nt_c(*args[:4], cp, args[4], m, n, k, wp, wb,
                                      _stream_handle(s, a.device))
    _check(st, "fp8bs_dense_nt_c")


def fp8bs_grouped_contiguous_nt_c(a, sfa, b, sfb, c, d, grouped_layout, workspace=None,
                                  stream=None):
    """Contiguous MoE layout with an FP32 addend c [m_total][n]."""
    args, m, n, k, g = _contiguous_args(a, sfa, b, sfb, d, grouped_layout)
    cp = _addend(c, d)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_CONTIGUOUS, m, n, k, g, 0, s, a.device)
        st = _load().fp8bs_grouped_contiguous_nt_c(*args[:4], cp, args[4], args[5], m, n, k, g,
                                                   wp, wb, _stream_handle(s, a.device))
    _check(st, "fp8bs_grouped_contiguous_nt_c")


def fp8bs_grouped_masked_nt_c(a, sfa, b, sfb, c, d, masked_m, expected_m: int = 0,
                              workspace=None, stream=None):
    """Masked MoE layout with an FP32 addend c [g][max_m][n]."""
    args, g, max_m, n, k = _masked_args(a, sfa, b, sfb, d, masked_m)
    cp = _addend(c, d)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_MASKED, max_m, n, k, g, int(expected_m), s,
                                   a.device)
        st = _load().fp8bs_grouped_masked_nt_c(*args[:4], cp, args[4], args[5], g, max_m,
                                               int(expected_m), n, k, wp, wb,
                                               _stream_handle(s, a.device))
    _check(st, "fp8bs_grouped_masked_nt_c")


# ---- stored forms nn / tn / tt and the K-grouped (weight-gradient) GEMM --------

def _dense_form(form, a, sfa, b, sfb, c, d, workspace, stream, e8=False):
    torch = _torch()
    a_t, b_t = form[0] == "t", form[1] == "t"
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    m, k = (a.shape[1], a.shape[0]) if a_t else (a.shape[0], a.shape[1])
    n, kb_ = (b.shape[0], b.shape[1]) if b_t else (b.shape[1], b.shape[0])
    if kb_ != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    kb = k // 128 if k % 128 == 0 else -1
    if e8:
        sap, sbp = _ue8m0_checks(sfa, sfb, 1, 1, m, n, k)
    else:
        sap = _dev_ptr(sfa, "sfa", (torch.float32,))
        sbp = _dev_ptr(sfb, "sfb", (torch.float32,))
        if kb > 0 and (sfa.numel() != kb * get_sfa_ld(m) or
                       sfb.numel() != ((n + 127) // 128) * kb):
            raise ValueError("scale tensor sizes do not match the shapes")
    args = (_dev_ptr(a, "a", _fp8_dtypes(), 2), sap, _dev_ptr(b, "b", _fp8_dtypes(), 2), sbp)
    dp = _dev_ptr(d, "d", _bf16_dtypes(), 2)
    cp = _addend(c, d) if c is not None else ctypes.c_void_p(None)
    code = {"nn": LAYOUT_DENSE_NN, "tn": LAYOUT_DENSE_TN, "tt": LAYOUT_DENSE_TT}[form]
    name = "fp8bs_dense_" + form + ("_ue8m0" if e8 else "")
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, code | (LAYOUT_UE8M0 if e8 else 0), m, n, k, 1, 0,
                                   s, a.device)
        st = getattr(_load(), name)(*args, cp, dp, m, n, k, wp, wb, _stream_handle(s, a.device))
    _check(st, name)


def fp8bs_dense_nn(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """D = bf16(C + A B): a e4m3 [m][k], b e4m3 [k][n] (N contiguous); scales and d as
    fp8bs_dense_nt; c optional FP32 [m][n]."""
    _dense_form("nn", a, sfa, b, sfb, c, d, workspace, stream)


def fp8bs_dense_tn(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """D = bf16(C + A^T B): a e4m3 [k][m], b e4m3 [k][n]."""
    _dense_form("tn", a, sfa, b, sfb, c, d, workspace, stream)


def fp8bs_dense_tt(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """D = bf16(C + A^T B^T): a e4m3 [k][m], b e4m3 [n][k]."""
    _dense_form("tt", a, sfa, b, sfb, c, d, workspace, stream)


def fp8bs_dense_nn_ue8m0(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """fp8bs_dense_nn with packed UE8M0 scales (sfa int32 [ceil(k/512)][ld(m)], sfb int32
    [ceil(n/128)][ceil(k/512)])."""
    _dense_form("nn", a, sfa, b, sfb, c, d, workspace, stream, e8=True)


def fp8bs_dense_tn_ue8m0(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """fp8bs_dense_tn with packed UE8M0 scales."""
    _dense_form("tn", a, sfa, b, sfb, c, d, workspace, stream, e8=True)


def fp8bs_dense_tt_ue8m0(a, sfa, b, sfb, d, c=None, workspace=None, stream=None):
    """fp8bs_dense_tt with packed UE8M0 scales."""
    _dense_form("tt", a, sfa, b, sfb, c, d, workspace, stream, e8=True)


def fp8bs_k_grouped_tn_contiguous_ue8m0(a, sfa, b, sfb, d, ks, c=None, workspace=None,
                                        stream=None):
    """K-grouped GEMM with packed UE8M0 scales: sfa int32 [ceil(k_total/512)][ld(m)], sfb
    int32 [ceil(k_total/512)][ld(n)] (``sfa_ue8m0_mn_major`` of the logical [m][k/128] /
    [n][k/128] power-of-two scales)."""
    _k_grouped(a, sfa, b, sfb, d, ks, c, workspace, stream, e8=True)


def fp8bs_k_grouped_tn_contiguous(a, sfa, b, sfb, d, ks, c=None, workspace=None, stream=None):
    """K-grouped weight-gradient GEMM: D[g] = C[g] + A_g^T B_g in FP32.

    a: e4m3 [k_total][m]; b: e4m3 [k_total][n]; sfa: f32 [k_total/128][ld(m)];
    sfb: f32 [k_total/128][ld(n)]; d: f32 [g][m][n] (every element written); ks: the g
    group sizes along K (a host sequence of ints, multiples of 128 adding up to k_total);
    c: optional f32 [g][m][n] (may be d itself)."""
    _k_grouped(a, sfa, b, sfb, d, ks, c, workspace, stream, e8=False)


def _k_grouped(a, sfa, b, sfb, d, ks, c, workspace, stream, e8):
    torch = _torch()
    sizes = [int(x) for x in ks]
    g = len(sizes)
    if a.dim() != 2 or b.dim() != 2 or d.dim() != 3:
        raise ValueError("a and b must be 2-D, d 3-D")
    k_total, m = a.shape
    n = b.shape[1]
    if b.shape[0] != k_total or tuple(d.shape) != (g, m, n):
        raise ValueError("shape mismatch between a, b, d and ks")
    kb = k_total // 128 if k_total % 128 == 0 else -1
    rows = (kb + 3) // 4 if e8 else kb                  # packed words: four chunks per int32
    sdt = torch.int32 if e8 else torch.float32
    args = (_dev_ptr(a, "a", _fp8_dtypes(), 2), _dev_ptr(sfa, "sfa", (sdt,)),
            _dev_ptr(b, "b", _fp8_dtypes(), 2), _dev_ptr(sfb, "sfb", (sdt,)))
    if kb >= 0 and (sfa.numel() != rows * get_sfa_ld(m) or sfb.numel() != rows * get_sfa_ld(n)):
        raise ValueError("scale tensor sizes do not match the shapes")
    dp = _dev_ptr(d, "d", (torch.float32,), 3)
    cp = _addend(c, d) if c is not None else ctypes.c_void_p(None)
    ks_host = (ctypes.c_int32 * max(g, 1))(*sizes)
    with _on_device(a):
        s = stream
        wp, wb, _keep = _workspace(workspace, LAYOUT_K_GROUPED | (LAYOUT_UE8M0 if e8 else 0), m,
                                   n, k_total, g, 0, s, a.device)
        name = "fp8bs_k_grouped_tn_contiguous" + ("_ue8m0" if e8 else "")
        st = getattr(_load(), name)(*args, cp, dp, ks_host, g, m, n, k_total, wp, wb,
                                    _stream_handle(s, a.device))
    _check(st, name)
