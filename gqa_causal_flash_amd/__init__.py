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

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")
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


def _dev(t, dtype, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes: int, device, workspace):
    import torch

    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
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
    st = lib().gqa_prefill_causal(_dev(q, torch.float16, "q"), _dev(k, torch.float16, "k"),
                                  _dev(v, torch.float16, "v"), _dev(o, torch.float16, "o"), nq, n_kv, q_pos0, hq, hkv,
                                  d, scale, None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                                  _stream(stream))
    _check(st, "gqa_prefill_causal")
    return o
