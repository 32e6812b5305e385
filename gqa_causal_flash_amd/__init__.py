"""Python binding of libgqa (causal grouped-query attention for MI355X).

Argument marshalling only: every function takes torch tensors (device memory
and the current stream come from PyTorch), checks dtype / shape / contiguity,
and calls the C entry point of the same name in libgqa.so.  All arithmetic
runs in the library's HIP kernels; there is no fallback path.  The library
must have been built (``python -m gqa_causal_flash_amd.build``); importing a
function that needs it raises ``GQAError`` when it is missing.
"""

from __future__ import annotations

import ctypes
import os

# GQA_LIBRARY names another build of the same library (e.g. a sanitizer build of its host code)
_LIB_PATH = os.environ.get("GQA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")
_lib = None

GQA_OK, GQA_ERR_INVALID, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = range(5)

# Entry points of include/gqa.h: name -> (restype, argtypes)
_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_szp = ctypes.POINTER(ctypes.c_size_t)
_i32p = ctypes.POINTER(ctypes.c_int32)
SIGNATURES = {
    "gqa_prefill_causal_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _szp]),
    "gqa_prefill_causal": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "gqa_prefill_paged_sparse_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _szp]),
    "gqa_prefill_paged_sparse": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    "gqa_prefill_paged_sparse_dropped": (_i32, [_vp, _i32p, _vp]),
    "gqa_verify_fp8kv_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _szp]),
    "gqa_verify_fp8kv": (_i32, [_vp, _vp, _vp, _f32, _f32, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "gqa_verify_fp8kv_noalloc": (_i32, [_vp, _vp, _vp, _f32, _f32, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "gqa_prefill_causal_e4m3": (_i32, [_vp, _f32, _vp, _f32, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                       _vp, _sz, _vp]),
    "gqa_prefill_causal_varlen_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "gqa_prefill_causal_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                         ctypes.c_float, _vp, ctypes.c_size_t, _vp]),
    "gqa_prefill_causal_varlen_skipped": (_i32, [_vp, _i32p, _vp]),
    "gqa_profile_start": (_i32, []),
    "gqa_profile_stop": (_i32, [ctypes.POINTER(ctypes.c_double), _i32p]),
    "gqa_profile_clock_mhz": (_i32, [ctypes.POINTER(ctypes.c_double)]),
    "gqa_status_string": (ctypes.c_char_p, [_i32]),
    "gqa_last_hip_error": (ctypes.c_int, []),
    "gqa_abi_version": (ctypes.c_int, []),
}


class GQAError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib().gqa_status_string(status).decode() if _lib is not None else f"status {status}"
        if status == GQA_ERR_HIP and _lib is not None:
            msg += f" (hipError {_lib.gqa_last_hip_error()})"
        super().__init__(f"{what}: {msg}" if what else msg)


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libgqa (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise GQAError(-1, f"libgqa.so not built at {_LIB_PATH}; run python -m gqa_causal_flash_amd.build")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            if not hasattr(l, name):
                continue
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int, what: str):
    if status != GQA_OK:
        raise GQAError(status, what)


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, shape=None):
    """Device pointer of a contiguous tensor of the given dtype (and shape, when given).

    The kernels size every buffer from the call's arguments, not from the
    allocation, so outputs and secondary inputs are checked against the shape
    those arguments imply before their pointers reach the library."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes: int, device, workspace):
    import torch

    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a tensor in device memory")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    return workspace, workspace.numel() * workspace.element_size()


# ------------------------------------------------------------- causal prefill
def gqa_prefill_causal_workspace_size(nq: int, n_kv: int, q_pos0: int, hq: int = 6, hkv: int = 1, d: int = 256) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d, ctypes.byref(out)),
           "gqa_prefill_causal_workspace_size")
    return out.value


def gqa_prefill_causal(q, k, v, q_pos0: int, scale: float, o=None, workspace=None, stream=None):
    """Dense causal GQA prefill; q [nq, Hq, D], k/v [n_kv, Hkv, D] fp16 -> o [nq, Hq, D]."""
    import torch

    nq, hq, d = q.shape
    n_kv, hkv, _ = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the same shape")
    if o is None:
        o = torch.empty_like(q)
    nbytes = gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d)
    ws, ws_bytes = _workspace(nbytes, q.device, workspace)
    st = lib().gqa_prefill_causal(_dev(q, torch.float16, "q"), _dev(k, torch.float16, "k", (n_kv, hkv, d)),
                                  _dev(v, torch.float16, "v"), _dev(o, torch.float16, "o", q.shape), nq, n_kv, q_pos0,
                                  hq, hkv, d, scale, None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                  _stream(stream))
    _check(st, "gqa_prefill_causal")
    return o


def gqa_prefill_causal_e4m3(q8, q_scale: float, k8, k_scale: float, v8, v_scale: float, q_pos0: int, scale: float,
                            o=None, workspace=None, stream=None):
    """Causal prefill over E4M3 codes; q8 [nq, Hq, D], k8/v8 [n_kv, Hkv, D] uint8 with one fp32 scale each
    -> o [nq, Hq, D] fp16."""
    import torch

    nq, hq, d = q8.shape
    n_kv, hkv, _ = k8.shape
    if tuple(v8.shape) != tuple(k8.shape):
        raise ValueError("k and v must have the same shape")
    if o is None:
        o = torch.empty((nq, hq, d), dtype=torch.float16, device=q8.device)
    nbytes = gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d)
    ws, ws_bytes = _workspace(nbytes, q8.device, workspace)
    st = lib().gqa_prefill_causal_e4m3(_dev(q8, torch.uint8, "q"), q_scale, _dev(k8, torch.uint8, "k", (n_kv, hkv, d)),
                                       k_scale, _dev(v8, torch.uint8, "v"), v_scale,
                                       _dev(o, torch.float16, "o", (nq, hq, d)), nq, n_kv,
                                       q_pos0, hq, hkv, d, scale,
                                       None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                       _stream(stream))
    _check(st, "gqa_prefill_causal_e4m3")
    return o


# --------------------------------------------------------------- varlen prefill
def gqa_prefill_causal_varlen_workspace_size(batch: int, total_q: int, hq: int = 6, hkv: int = 1, d: int = 256) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().gqa_prefill_causal_varlen_workspace_size(batch, total_q, hq, hkv, d, ctypes.byref(out)),
           "gqa_prefill_causal_varlen_workspace_size")
    return out.value


def gqa_prefill_causal_varlen(q, k, v, cu_q, cu_kv, scale: float, o=None, lse=None, want_lse: bool = True,
                              workspace=None, stream=None):
    """Causal prefill of a packed batch; q [total_q, Hq, D], k/v [total_kv, Hkv, D] fp16, cu_q/cu_kv int32
    [batch + 1] on device -> (o [total_q, Hq, D], lse [total_q, Hq] fp32 or None)."""
    import torch

    total_q, hq, d = q.shape
    total_kv, hkv, _ = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the same shape")
    batch = cu_q.numel() - 1
    if cu_kv.numel() != batch + 1:
        raise ValueError("cu_q and cu_kv must have the same length")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    nbytes = gqa_prefill_causal_varlen_workspace_size(batch, total_q, hq, hkv, d)
    ws, ws_bytes = _workspace(nbytes, q.device, workspace)
    st = lib().gqa_prefill_causal_varlen(
        _dev(q, torch.float16, "q"), _dev(k, torch.float16, "k", (total_kv, hkv, d)), _dev(v, torch.float16, "v"),
        _dev(o, torch.float16, "o", q.shape), None if lse is None else _dev(lse, torch.float32, "lse", (total_q, hq)),
        _dev(cu_q, torch.int32, "cu_q", (batch + 1,)), _dev(cu_kv, torch.int32, "cu_kv", (batch + 1,)), batch, total_q,
        total_kv, hq, hkv, d,
        scale, ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream(stream))
    _check(st, "gqa_prefill_causal_varlen")
    return o, lse, ws


def gqa_prefill_causal_varlen_skipped(workspace, stream=None) -> int:
    """Sequences the last varlen call on `workspace` skipped as invalid (synchronises the stream)."""
    n = ctypes.c_int32(0)
    _check(lib().gqa_prefill_causal_varlen_skipped(_dev(workspace, None, "workspace"), ctypes.byref(n),
                                                   _stream(stream)), "gqa_prefill_causal_varlen_skipped")
    return n.value


# --------------------------------------------------------------- kernel timing
def gqa_profile_start():
    _check(lib().gqa_profile_start(), "gqa_profile_start")


def gqa_profile_stop():
    """(total_ms, count) of the main attention kernels launched since gqa_profile_start()."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(lib().gqa_profile_stop(ctypes.byref(ms), ctypes.byref(n)), "gqa_profile_stop")
    return ms.value, n.value


def gqa_profile_clock_mhz():
    """Average shader clock (MHz) of the dense prefill kernels of the last stopped profiling session (0 if none)."""
    mhz = ctypes.c_double(0.0)
    _check(lib().gqa_profile_clock_mhz(ctypes.byref(mhz)), "gqa_profile_clock_mhz")
    return mhz.value


# ------------------------------------------------------ paged block-sparse
def gqa_prefill_paged_sparse_workspace_size(nq: int, n_block_ids: int, qblock_rows: int = 64, kv_block_tokens: int = 4,
                                            hq: int = 6, hkv: int = 1, d: int = 256) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().gqa_prefill_paged_sparse_workspace_size(nq, n_block_ids, qblock_rows, kv_block_tokens, hq, hkv, d,
                                                         ctypes.byref(out)), "gqa_prefill_paged_sparse_workspace_size")
    return out.value


def gqa_prefill_paged_sparse(q, k_cache, v_cache, page_table, qblock_offsets, kv_block_ids, q_pos0: int,
                             live_len: int, scale: float, qblock_rows: int = 64, kv_block_tokens: int = 4, o=None,
                             workspace=None, stream=None):
    """Paged block-sparse causal prefill; caches [n_pages, page_size, Hkv, D] fp16, index arrays int32 on device."""
    import torch

    nq, hq, d = q.shape
    n_pages, page_size, hkv, _ = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must have the same shape")
    n_ids = kv_block_ids.numel()
    if o is None:
        o = torch.empty_like(q)
    nbytes = gqa_prefill_paged_sparse_workspace_size(nq, n_ids, qblock_rows, kv_block_tokens, hq, hkv, d)
    ws, ws_bytes = _workspace(nbytes, q.device, workspace)
    n_qblocks = -(-nq // qblock_rows) if qblock_rows > 0 else 0
    st = lib().gqa_prefill_paged_sparse(
        _dev(q, torch.float16, "q"), _dev(k_cache, torch.float16, "k_cache", (n_pages, page_size, hkv, d)),
        _dev(v_cache, torch.float16, "v_cache"),
        _dev(page_table, torch.int32, "page_table", (page_table.numel(),)), page_table.numel(), n_pages, page_size,
        _dev(qblock_offsets, torch.int32, "qblock_offsets", (n_qblocks + 1,)),
        _dev(kv_block_ids, torch.int32, "kv_block_ids", (n_ids,)) if n_ids else None, n_ids, qblock_rows,
        kv_block_tokens, nq, q_pos0, live_len, hq, hkv, d, scale, _dev(o, torch.float16, "o", q.shape),
        None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream(stream))
    _check(st, "gqa_prefill_paged_sparse")
    return o, ws


def gqa_prefill_paged_sparse_dropped(workspace, stream=None) -> int:
    """Index entries the last paged call on `workspace` dropped as invalid (synchronises the stream)."""
    n = ctypes.c_int32(0)
    _check(lib().gqa_prefill_paged_sparse_dropped(_dev(workspace, None, "workspace"), ctypes.byref(n),
                                                  _stream(stream)), "gqa_prefill_paged_sparse_dropped")
    return n.value


# ------------------------------------------------------------ FP8 verifier
def gqa_verify_fp8kv_workspace_size(nq: int, n_kv: int, hq: int = 6, hkv: int = 1, d: int = 256) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().gqa_verify_fp8kv_workspace_size(nq, n_kv, hq, hkv, d, ctypes.byref(out)),
           "gqa_verify_fp8kv_workspace_size")
    return out.value


def gqa_verify_fp8kv(q, k_e4m3, v_e4m3, k_scale: float, v_scale: float, scale: float, o=None, workspace=None,
                     stream=None):
    """Causal verifier tail: q [nq, Hq, D] fp16 at the last nq positions; k/v [n_kv, Hkv, D] uint8 E4M3 codes."""
    import torch

    nq, hq, d = q.shape
    n_kv, hkv, _ = k_e4m3.shape
    if tuple(v_e4m3.shape) != tuple(k_e4m3.shape):
        raise ValueError("k and v must have the same shape")
    if o is None:
        o = torch.empty_like(q)
    nbytes = gqa_verify_fp8kv_workspace_size(nq, n_kv, hq, hkv, d)
    ws, ws_bytes = _workspace(nbytes, q.device, workspace)
    st = lib().gqa_verify_fp8kv(_dev(q, torch.float16, "q"), _dev(k_e4m3, torch.uint8, "k_e4m3", (n_kv, hkv, d)),
                                _dev(v_e4m3, torch.uint8, "v_e4m3"), k_scale, v_scale,
                                _dev(o, torch.float16, "o", q.shape), nq,
                                n_kv, hq, hkv, d, scale, None if ws is None else ctypes.c_void_p(ws.data_ptr()),
                                ws_bytes, _stream(stream))
    _check(st, "gqa_verify_fp8kv")
    return o


def gqa_verify_fp8kv_noalloc(q, k_e4m3, v_e4m3, k_scale: float, v_scale: float, scale: float, o=None, stream=None):
    """gqa_verify_fp8kv without a workspace: the library's fixed per-device scratch holds the partials, and the
    C call allocates nothing (pass `o` to allocate nothing here either).  Calls on one device must not overlap."""
    import torch

    nq, hq, d = q.shape
    n_kv, hkv, _ = k_e4m3.shape
    if tuple(v_e4m3.shape) != tuple(k_e4m3.shape):
        raise ValueError("k and v must have the same shape")
    if o is None:
        o = torch.empty_like(q)
    st = lib().gqa_verify_fp8kv_noalloc(_dev(q, torch.float16, "q"),
                                        _dev(k_e4m3, torch.uint8, "k_e4m3", (n_kv, hkv, d)),
                                        _dev(v_e4m3, torch.uint8, "v_e4m3"), k_scale, v_scale,
                                        _dev(o, torch.float16, "o", q.shape), nq, n_kv, hq, hkv, d, scale,
                                        _stream(stream))
    _check(st, "gqa_verify_fp8kv_noalloc")
    return o
