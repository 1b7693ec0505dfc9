"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h and
include/fp8_fp4_gemm.h).

Argument marshalling only: every function passes device pointers, sizes and a HIP
stream to the library and raises MoEError on a non-zero status. Tensors are torch
tensors used as device memory; nothing here computes any part of the forward.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_TOKENS = -5
MOE_ERR_HIP = -6
MOE_ERR_SCRATCH = -7

EXPORTED = ("moe_packed_weights_bytes", "moe_prepare_weights", "moe_workspace_bytes",
            "moe_forward", "moe_forward_events", "moe_forward_noalloc", "moe_workspace_layout", "moe_read_diagnostics",
            "moe_status_string", "moe_version",
            "moe_gemm_packed_b_bytes", "moe_gemm_prepare_b", "moe_gemm_workspace_bytes",
            "moe_fp8_fp4_gemm", "moe_m_grouped_fp8_fp4_gemm_contiguous",
            "moe_m_grouped_fp8_fp4_gemm_masked", "moe_cast_to_fp8")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")


class moe_shape_t(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32)]


class moe_layout_t(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("max_tiles", ctypes.c_int32),
                ("meta", ctypes.c_size_t), ("counts", ctypes.c_size_t),
                ("offsets", ctypes.c_size_t), ("perm", ctypes.c_size_t),
                ("inv", ctypes.c_size_t), ("tile_expert", ctypes.c_size_t),
                ("tile_row0", ctypes.c_size_t), ("h8", ctypes.c_size_t),
                ("h_sf", ctypes.c_size_t), ("h_sf_stride", ctypes.c_size_t),
                ("stage", ctypes.c_size_t), ("xg", ctypes.c_size_t),
                ("xg_sf", ctypes.c_size_t), ("total", ctypes.c_size_t)]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m block_scaled_fp8_dispatch_amd.build`; "
                          "the MoE forward has no other implementation")
    lib = ctypes.CDLL(path)
    P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    shp = ctypes.POINTER(moe_shape_t)
    lib.moe_packed_weights_bytes.argtypes = [shp]
    lib.moe_packed_weights_bytes.restype = S
    lib.moe_prepare_weights.argtypes = [shp, P, P, P, P, P, S, P]
    lib.moe_prepare_weights.restype = ctypes.c_int
    lib.moe_workspace_bytes.argtypes = [shp]
    lib.moe_workspace_bytes.restype = S
    lib.moe_forward.argtypes = [P, P, P, P, P, I32, shp, P, P, S, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_events.argtypes = [P, P, P, P, P, I32, shp, P, P, S, P, ctypes.POINTER(P)]
    lib.moe_forward_events.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [P, P, P, P, P, I32, shp, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_workspace_layout.argtypes = [shp, I32, ctypes.POINTER(moe_layout_t)]
    lib.moe_workspace_layout.restype = ctypes.c_int
    lib.moe_read_diagnostics.argtypes = [shp, P, ctypes.POINTER(I32), ctypes.POINTER(I32), P]
    lib.moe_read_diagnostics.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_int
    lib.moe_gemm_packed_b_bytes.argtypes = [I32, I32, I32]
    lib.moe_gemm_packed_b_bytes.restype = S
    lib.moe_gemm_prepare_b.argtypes = [I32, I32, I32, P, P, P, S, P]
    lib.moe_gemm_prepare_b.restype = ctypes.c_int
    lib.moe_gemm_workspace_bytes.argtypes = [I32, I32]
    lib.moe_gemm_workspace_bytes.restype = S
    lib.moe_fp8_fp4_gemm.argtypes = [P, P, P, I32, I32, I32, P, P, S, P]
    lib.moe_fp8_fp4_gemm.restype = ctypes.c_int
    lib.moe_m_grouped_fp8_fp4_gemm_contiguous.argtypes = [P, P, P, P, I32, I32, I32, I32, P, P, S, P]
    lib.moe_m_grouped_fp8_fp4_gemm_contiguous.restype = ctypes.c_int
    lib.moe_m_grouped_fp8_fp4_gemm_masked.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, P, S, P]
    lib.moe_m_grouped_fp8_fp4_gemm_masked.restype = ctypes.c_int
    lib.moe_cast_to_fp8.argtypes = [P, I32, I32, P, P, P]
    lib.moe_cast_to_fp8.restype = ctypes.c_int
    _lib = lib
    return lib


def make_shape(num_experts: int, hidden: int, intermediate: int, num_topk: int,
               max_tokens: int) -> moe_shape_t:
    return moe_shape_t(num_experts, hidden, intermediate, num_topk, max_tokens)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_version() -> int:
    return load_library().moe_version()


def moe_packed_weights_bytes(shape: moe_shape_t) -> int:
    return load_library().moe_packed_weights_bytes(ctypes.byref(shape))


def moe_workspace_bytes(shape: moe_shape_t) -> int:
    return load_library().moe_workspace_bytes(ctypes.byref(shape))


def moe_prepare_weights(shape: moe_shape_t, w1, w1_sf, w2, w2_sf, packed, stream=None) -> None:
    st = load_library().moe_prepare_weights(
        ctypes.byref(shape), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf), _ptr(packed),
        packed.numel() * packed.element_size(), _stream(stream))
    _check(st, "moe_prepare_weights")


def moe_forward(y, x_fp8, x_sf, topk_idx, topk_weights, num_tokens: int, shape: moe_shape_t,
                packed, workspace, stream=None) -> None:
    st = load_library().moe_forward(
        _ptr(y), _ptr(x_fp8), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_weights), int(num_tokens),
        ctypes.byref(shape), _ptr(packed), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_forward")


def moe_forward_events(y, x_fp8, x_sf, topk_idx, topk_weights, num_tokens: int,
                       shape: moe_shape_t, packed, workspace, events, stream=None) -> None:
    """moe_forward that also records 5 torch.cuda.Event objects at the stage boundaries
    (before dispatch, after dispatch, after Linear1, after Linear2, after the combine)."""
    handles = (ctypes.c_void_p * 5)(*[_event_handle(e) for e in events])
    st = load_library().moe_forward_events(
        _ptr(y), _ptr(x_fp8), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_weights), int(num_tokens),
        ctypes.byref(shape), _ptr(packed), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), handles)
    _check(st, "moe_forward_events")


# Bytes of the library's fixed scratch array (MOE_NOALLOC_SCRATCH_BYTES in include/moe.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(y, x_fp8, x_sf, topk_idx, topk_weights, num_tokens: int,
                        shape: moe_shape_t, packed, stream=None) -> None:
    """moe_forward with its workspace in the library's fixed per-GPU scratch array (no
    workspace argument; calls on one GPU must not overlap)."""
    st = load_library().moe_forward_noalloc(
        _ptr(y), _ptr(x_fp8), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_weights), int(num_tokens),
        ctypes.byref(shape), _ptr(packed), _stream(stream))
    _check(st, "moe_forward_noalloc")


def moe_forward_noalloc_raw(y_ptr, x_ptr, xsf_ptr, idx_ptr, w_ptr, num_tokens, shape, packed_ptr,
                            stream_ptr) -> int:
    """Unchecked call with raw integer pointers; returns the status (for error-path tests)."""
    return load_library().moe_forward_noalloc(y_ptr, x_ptr, xsf_ptr, idx_ptr, w_ptr, int(num_tokens),
                                              ctypes.byref(shape), packed_ptr, stream_ptr)


def _event_handle(ev) -> int:
    if isinstance(ev, int):
        return ev
    h = ev.cuda_event
    if not h:
        # torch creates the HIP event lazily, on its first record
        import torch
        ev.record(torch.cuda.current_stream())
        h = ev.cuda_event
    return h


def moe_forward_raw(y_ptr, x_ptr, xsf_ptr, idx_ptr, w_ptr, num_tokens, shape, packed_ptr,
                    ws_ptr, ws_bytes, stream_ptr) -> int:
    """Unchecked call with raw integer pointers; returns the status (for error-path tests)."""
    return load_library().moe_forward(y_ptr, x_ptr, xsf_ptr, idx_ptr, w_ptr, int(num_tokens),
                                      ctypes.byref(shape), packed_ptr, ws_ptr, ws_bytes, stream_ptr)


def moe_prepare_weights_raw(shape, w1, w1_sf, w2, w2_sf, packed, packed_bytes, stream) -> int:
    return load_library().moe_prepare_weights(ctypes.byref(shape), w1, w1_sf, w2, w2_sf, packed,
                                              packed_bytes, stream)


def moe_workspace_layout(shape: moe_shape_t, num_tokens: int) -> dict:
    out = moe_layout_t()
    _check(load_library().moe_workspace_layout(ctypes.byref(shape), int(num_tokens),
                                               ctypes.byref(out)), "moe_workspace_layout")
    return {name: getattr(out, name) for name, _ in moe_layout_t._fields_}


def moe_read_diagnostics(shape: moe_shape_t, workspace, stream=None):
    inv = ctypes.c_int32(0)
    counts = (ctypes.c_int32 * shape.num_experts)()
    _check(load_library().moe_read_diagnostics(ctypes.byref(shape), _ptr(workspace),
                                               ctypes.byref(inv), counts, _stream(stream)),
           "moe_read_diagnostics")
    return inv.value, list(counts)


# ---------------------------------------------------------------------------
# FP8 x FP4 GEMMs and the FP8 cast (include/fp8_fp4_gemm.h)
# ---------------------------------------------------------------------------


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def moe_gemm_packed_b_bytes(groups: int, n: int, k: int) -> int:
    return load_library().moe_gemm_packed_b_bytes(int(groups), int(n), int(k))


def moe_gemm_prepare_b(groups: int, n: int, k: int, b, b_sf, packed, stream=None) -> None:
    _check(load_library().moe_gemm_prepare_b(int(groups), int(n), int(k), _ptr(b), _ptr(b_sf),
                                             _ptr(packed), _nbytes(packed), _stream(stream)),
           "moe_gemm_prepare_b")


def moe_gemm_workspace_bytes(max_rows: int, groups: int) -> int:
    return load_library().moe_gemm_workspace_bytes(int(max_rows), int(groups))


def moe_fp8_fp4_gemm(d, a, a_sf, m: int, n: int, k: int, packed_b, workspace, stream=None) -> None:
    _check(load_library().moe_fp8_fp4_gemm(_ptr(d), _ptr(a), _ptr(a_sf), int(m), int(n), int(k),
                                           _ptr(packed_b), _ptr(workspace), _nbytes(workspace),
                                           _stream(stream)), "moe_fp8_fp4_gemm")


def moe_m_grouped_fp8_fp4_gemm_contiguous(d, a, a_sf, group_of_row, m: int, groups: int, n: int,
                                          k: int, packed_b, workspace, stream=None) -> None:
    _check(load_library().moe_m_grouped_fp8_fp4_gemm_contiguous(
        _ptr(d), _ptr(a), _ptr(a_sf), _ptr(group_of_row), int(m), int(groups), int(n), int(k),
        _ptr(packed_b), _ptr(workspace), _nbytes(workspace), _stream(stream)),
        "moe_m_grouped_fp8_fp4_gemm_contiguous")


def moe_m_grouped_fp8_fp4_gemm_masked(d, a, a_sf, masked_m, groups: int, max_m: int,
                                      expected_m: int, n: int, k: int, packed_b, workspace,
                                      stream=None) -> None:
    _check(load_library().moe_m_grouped_fp8_fp4_gemm_masked(
        _ptr(d), _ptr(a), _ptr(a_sf), _ptr(masked_m), int(groups), int(max_m), int(expected_m),
        int(n), int(k), _ptr(packed_b), _ptr(workspace), _nbytes(workspace), _stream(stream)),
        "moe_m_grouped_fp8_fp4_gemm_masked")


def moe_cast_to_fp8(x, rows: int, cols: int, x_fp8, x_sf, stream=None) -> None:
    _check(load_library().moe_cast_to_fp8(_ptr(x), int(rows), int(cols), _ptr(x_fp8), _ptr(x_sf),
                                          _stream(stream)), "moe_cast_to_fp8")


def gemm_call_raw(name: str, *args) -> int:
    """Unchecked call of one of the GEMM / cast entry points with raw arguments; returns the
    status (for error-path tests)."""
    return getattr(load_library(), name)(*args)
