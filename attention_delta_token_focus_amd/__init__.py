"""Python binding of libfocus, the FOCUS eviction hot path on MI355X.

Each function has the name and the parameter order of the C entry point
declared in include/focus.h. Pointer parameters take contiguous torch CUDA
tensors (or None where the C call allows NULL); `stream` takes None (torch's
current stream), a torch.cuda.Stream or a raw hipStream_t integer. This
module only marshals arguments: every step runs in the HIP kernels of
libfocus.so, and importing it fails if that library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "FOCUS_OK", "FOCUS_ERR_INVALID_ARG", "FOCUS_ERR_UNSUPPORTED",
    "FOCUS_ERR_WORKSPACE", "FOCUS_ERR_HIP", "FOCUS_F32", "FOCUS_BF16",
    "FOCUS_KEEP_PREDECESSOR", "FOCUS_KEEP_MASKED_PREFIX",
    "FocusError", "lib", "lib_path", "dtype_code", "focus_version",
    "focus_status_string", "focus_last_error", "focus_schedule",
    "focus_block_attn_importance_workspace", "focus_block_attn_importance",
    "focus_block_attn_importance_paged", "focus_block_attn_importance_noalloc",
    "focus_delta_topk", "focus_compact", "focus_select", "focus_select_masked",
    "focus_select_dynamic",
    "focus_retained_attn_workspace", "focus_retained_attn",
    "focus_retained_attn_paged",
]

FOCUS_OK = 0
FOCUS_ERR_INVALID_ARG = 1
FOCUS_ERR_UNSUPPORTED = 2
FOCUS_ERR_WORKSPACE = 3
FOCUS_ERR_HIP = 4
FOCUS_F32 = 0
FOCUS_BF16 = 1
FOCUS_KEEP_PREDECESSOR = 1
FOCUS_KEEP_MASKED_PREFIX = 2

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "lib", "libfocus.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"libfocus is not built ({lib_path} missing); build it with "
        "`python attention_delta_token_focus_amd/build.py`")

_c = ctypes
_P = _c.c_void_p
_I = _c.c_int
_SZ = _c.c_size_t

lib = _c.CDLL(lib_path)
_SIGS = {
    "focus_version": (_c.c_char_p, []),
    "focus_status_string": (_c.c_char_p, [_I]),
    "focus_last_error": (_c.c_char_p, []),
    "focus_block_attn_importance_workspace": (
        _I, [_I, _I, _I, _I, _I, _I, _c.POINTER(_SZ)]),
    "focus_schedule": (_I, [_I, _P, _P, _P]),
    "focus_block_attn_importance": (
        _I, [_I, _I, _I, _I, _I, _I, _c.c_float, _P, _P, _P, _P, _P, _P, _P,
             _I, _P, _P, _P, _P, _SZ, _P]),
    "focus_block_attn_importance_paged": (
        _I, [_I, _I, _I, _I, _I, _I, _c.c_float, _P, _P, _P, _P, _P, _P, _I,
             _I, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "focus_block_attn_importance_noalloc": (
        _I, [_I, _I, _I, _I, _I, _I, _c.c_float, _P, _P, _P, _P, _P, _P, _I,
             _P, _P, _P, _P]),
    "focus_delta_topk": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "focus_compact": (_I, [_I, _I, _P, _P, _P, _P]),
    "focus_select": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "focus_select_masked": (
        _I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P]),
    "focus_select_dynamic": (
        _I, [_I, _I, _I, _I, _P, _P, _P, _P, _c.c_float, _I, _P, _P, _P, _P, _P,
             _P, _P]),
    "focus_retained_attn_workspace": (
        _I, [_I, _I, _I, _I, _I, _I, _I, _c.POINTER(_SZ)]),
    "focus_retained_attn": (
        _I, [_I, _I, _I, _I, _I, _I, _c.c_float, _P, _P, _P, _P, _P, _I, _I,
             _P, _P, _P, _P, _I, _P, _P, _SZ, _P]),
    "focus_retained_attn_paged": (
        _I, [_I, _I, _I, _I, _I, _I, _c.c_float, _P, _P, _P, _P, _P, _I, _I,
             _P, _P, _P, _I, _I, _P, _P, _I, _P, _P, _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class FocusError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{focus_status_string(status)}: {message}")
        self.status = status


def focus_version() -> str:
    return lib.focus_version().decode()


def focus_status_string(status: int) -> str:
    return lib.focus_status_string(int(status)).decode()


def focus_last_error() -> str:
    return lib.focus_last_error().decode()


def dtype_code(dt) -> int:
    if dt in (FOCUS_F32, FOCUS_BF16) and isinstance(dt, int):
        return dt
    if dt == torch.bfloat16:
        return FOCUS_BF16
    if dt == torch.float32:
        return FOCUS_F32
    raise ValueError(f"libfocus supports bfloat16 and float32, not {dt}")


def _ptr(t, name: str, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int) -> None:
    if status != FOCUS_OK:
        raise FocusError(status, focus_last_error())


def focus_block_attn_importance_workspace(batch, B, Hq, Hkv, d,
                                          max_prefix) -> int:
    n = _SZ(0)
    _check(lib.focus_block_attn_importance_workspace(
        batch, B, Hq, Hkv, d, max_prefix, _c.byref(n)))
    return n.value


def focus_schedule(batch, cu_prefix, order, stream=None) -> None:
    _check(lib.focus_schedule(batch, _ptr(cu_prefix, "cu_prefix"),
                              _ptr(order, "order"), _stream(stream)))


def focus_block_attn_importance(dt, batch, B, Hq, Hkv, d, scale, q, k_blk,
                                v_blk, k_cache, v_cache, cu_prefix, order,
                                max_prefix, out, imp, lse=None,
                                workspace=None, workspace_bytes=0,
                                stream=None) -> None:
    _check(lib.focus_block_attn_importance(
        dtype_code(dt), batch, B, Hq, Hkv, d, float(scale),
        _ptr(q, "q"), _ptr(k_blk, "k_blk"), _ptr(v_blk, "v_blk", True),
        _ptr(k_cache, "k_cache", True), _ptr(v_cache, "v_cache", True),
        _ptr(cu_prefix, "cu_prefix"), _ptr(order, "order", True),
        max_prefix, _ptr(out, "out", True),
        _ptr(imp, "imp"), _ptr(lse, "lse", True),
        _ptr(workspace, "workspace", True), workspace_bytes,
        _stream(stream)))


def focus_block_attn_importance_noalloc(dt, batch, B, Hq, Hkv, d, scale, q,
                                        k_blk, v_blk, k_cache, v_cache,
                                        cu_prefix, max_prefix, out, imp,
                                        lse=None, stream=None) -> None:
    _check(lib.focus_block_attn_importance_noalloc(
        dtype_code(dt), batch, B, Hq, Hkv, d, float(scale),
        _ptr(q, "q"), _ptr(k_blk, "k_blk"), _ptr(v_blk, "v_blk", True),
        _ptr(k_cache, "k_cache", True), _ptr(v_cache, "v_cache", True),
        _ptr(cu_prefix, "cu_prefix"), max_prefix, _ptr(out, "out", True),
        _ptr(imp, "imp"), _ptr(lse, "lse", True), _stream(stream)))


def focus_block_attn_importance_paged(dt, batch, B, Hq, Hkv, d, scale, q,
                                      k_blk, v_blk, k_pages, v_pages,
                                      page_table, page_size, pages_per_seq,
                                      cu_prefix, order, max_prefix, out, imp,
                                      lse=None, workspace=None,
                                      workspace_bytes=0, stream=None) -> None:
    _check(lib.focus_block_attn_importance_paged(
        dtype_code(dt), batch, B, Hq, Hkv, d, float(scale),
        _ptr(q, "q"), _ptr(k_blk, "k_blk"), _ptr(v_blk, "v_blk", True),
        _ptr(k_pages, "k_pages", True), _ptr(v_pages, "v_pages", True),
        _ptr(page_table, "page_table", True), page_size, pages_per_seq,
        _ptr(cu_prefix, "cu_prefix"), _ptr(order, "order", True),
        max_prefix, _ptr(out, "out", True),
        _ptr(imp, "imp"), _ptr(lse, "lse", True),
        _ptr(workspace, "workspace", True), workspace_bytes,
        _stream(stream)))


def focus_delta_topk(batch, B, Hq, pool_k, imp0, imp1, k_keep, keep,
                     dI=None, stream=None) -> None:
    _check(lib.focus_delta_topk(
        batch, B, Hq, pool_k, _ptr(imp0, "imp0"), _ptr(imp1, "imp1"),
        _ptr(k_keep, "k_keep"), _ptr(keep, "keep"), _ptr(dI, "dI", True),
        _stream(stream)))


def focus_compact(batch, B, keep, idx, cu_ret, stream=None) -> None:
    _check(lib.focus_compact(batch, B, _ptr(keep, "keep"), _ptr(idx, "idx"),
                             _ptr(cu_ret, "cu_ret"), _stream(stream)))


def focus_select(batch, B, Hq, pool_k, imp0, imp1, k_keep, keep, dI, idx,
                 cu_ret, stream=None) -> None:
    _check(lib.focus_select(
        batch, B, Hq, pool_k, _ptr(imp0, "imp0"), _ptr(imp1, "imp1"),
        _ptr(k_keep, "k_keep"), _ptr(keep, "keep"), _ptr(dI, "dI", True),
        _ptr(idx, "idx"), _ptr(cu_ret, "cu_ret"), _stream(stream)))


def focus_select_masked(batch, B, Hq, pool_k, imp0, imp1, masked, k_keep,
                        rules, keep, cand=None, dI=None, idx=None, cu_ret=None,
                        stream=None) -> None:
    _check(lib.focus_select_masked(
        batch, B, Hq, pool_k, _ptr(imp0, "imp0"), _ptr(imp1, "imp1"),
        _ptr(masked, "masked", True), _ptr(k_keep, "k_keep"), int(rules),
        _ptr(keep, "keep"), _ptr(cand, "cand", True), _ptr(dI, "dI", True),
        _ptr(idx, "idx", True), _ptr(cu_ret, "cu_ret", True), _stream(stream)))


def focus_select_dynamic(batch, B, Hq, pool_k, imp0, imp1, masked, yield_hist,
                         alpha, rules, keep, k_used=None, cand=None, dI=None,
                         idx=None, cu_ret=None, stream=None) -> None:
    _check(lib.focus_select_dynamic(
        batch, B, Hq, pool_k, _ptr(imp0, "imp0"), _ptr(imp1, "imp1"),
        _ptr(masked, "masked", True), _ptr(yield_hist, "yield_hist"),
        float(alpha), int(rules), _ptr(k_used, "k_used", True),
        _ptr(keep, "keep"), _ptr(cand, "cand", True), _ptr(dI, "dI", True),
        _ptr(idx, "idx", True), _ptr(cu_ret, "cu_ret", True), _stream(stream)))


def focus_retained_attn_workspace(batch, Hq, Hkv, d, max_prefix, n_ret,
                                  max_ret) -> int:
    n = _SZ(0)
    _check(lib.focus_retained_attn_workspace(
        batch, Hq, Hkv, d, max_prefix, n_ret, max_ret, _c.byref(n)))
    return n.value


def focus_retained_attn(dt, batch, B, Hq, Hkv, d, scale, q_src, k_src,
                        v_src, idx, cu_ret, n_ret, max_ret, k_cache, v_cache,
                        cu_prefix, order, max_prefix, out, workspace=None,
                        workspace_bytes=0, stream=None) -> None:
    _check(lib.focus_retained_attn(
        dtype_code(dt), batch, B, Hq, Hkv, d, float(scale),
        _ptr(q_src, "q_src"), _ptr(k_src, "k_src"), _ptr(v_src, "v_src"),
        _ptr(idx, "idx", n_ret == 0), _ptr(cu_ret, "cu_ret", n_ret == 0),
        n_ret, max_ret, _ptr(k_cache, "k_cache", True),
        _ptr(v_cache, "v_cache", True), _ptr(cu_prefix, "cu_prefix"),
        _ptr(order, "order", True), max_prefix, _ptr(out, "out", n_ret == 0),
        _ptr(workspace, "workspace", True), workspace_bytes,
        _stream(stream)))


def focus_retained_attn_paged(dt, batch, B, Hq, Hkv, d, scale, q_src, k_src,
                              v_src, idx, cu_ret, n_ret, max_ret, k_pages,
                              v_pages, page_table, page_size, pages_per_seq,
                              cu_prefix, order, max_prefix, out,
                              workspace=None, workspace_bytes=0,
                              stream=None) -> None:
    _check(lib.focus_retained_attn_paged(
        dtype_code(dt), batch, B, Hq, Hkv, d, float(scale),
        _ptr(q_src, "q_src"), _ptr(k_src, "k_src"), _ptr(v_src, "v_src"),
        _ptr(idx, "idx", n_ret == 0), _ptr(cu_ret, "cu_ret", n_ret == 0),
        n_ret, max_ret, _ptr(k_pages, "k_pages", True),
        _ptr(v_pages, "v_pages", True), _ptr(page_table, "page_table", True),
        page_size, pages_per_seq, _ptr(cu_prefix, "cu_prefix"),
        _ptr(order, "order", True), max_prefix, _ptr(out, "out", n_ret == 0),
        _ptr(workspace, "workspace", True), workspace_bytes,
        _stream(stream)))
