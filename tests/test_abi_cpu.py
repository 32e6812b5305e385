"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no GPU needed)."""

import ctypes
import os
import re

import pytest

import gqa_causal_flash_amd as g

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gqa.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = g.lib()
    names = declared_symbols()
    assert "gqa_prefill_causal" in names and len(names) >= 10
    missing = [n for n in names if not hasattr(lib, n)]
    assert missing == []
    assert set(names) <= set(g.SIGNATURES)


def test_abi_version_and_status_strings():
    lib = g.lib()
    assert lib.gqa_abi_version() == 1
    for s in range(5):
        assert lib.gqa_status_string(s).startswith(b"GQA_")
    assert lib.gqa_last_hip_error() == 0


def _ws(nq, n_kv, q_pos0, hq=6, hkv=1, d=256):
    out = ctypes.c_size_t(0)
    st = g.lib().gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d, ctypes.byref(out))
    return st, out.value


def test_prefill_workspace_query():
    st, n = _ws(8000, 128000, 120000)
    assert st == g.GQA_OK and n > 0
    assert _ws(1, 1, 0) == (g.GQA_OK, 0)
    assert _ws(0, 10, 0)[0] == g.GQA_ERR_INVALID
    assert _ws(10, 10, 1)[0] == g.GQA_ERR_INVALID        # q_pos0 + nq > n_kv
    assert _ws(10, 10, 0, hq=8)[0] == g.GQA_ERR_UNSUPPORTED
    assert _ws(10, 10, 0, d=128)[0] == g.GQA_ERR_UNSUPPORTED
    assert _ws(10, 10, 0, hq=12, hkv=2)[0] == g.GQA_ERR_UNSUPPORTED
    assert g.lib().gqa_prefill_causal_workspace_size(1, 1, 0, 6, 1, 256, None) == g.GQA_ERR_INVALID


def _prefill(q=FAKE, k=FAKE, v=FAKE, o=FAKE, nq=8000, n_kv=128000, q_pos0=120000, hq=6, hkv=1, d=256,
             scale=0.0625, ws=None, ws_bytes=0):
    return g.lib().gqa_prefill_causal(q, k, v, o, nq, n_kv, q_pos0, hq, hkv, d, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), g.GQA_ERR_INVALID),
    (dict(o=None), g.GQA_ERR_INVALID),
    (dict(nq=-1), g.GQA_ERR_INVALID),
    (dict(q_pos0=-1), g.GQA_ERR_INVALID),
    (dict(q_pos0=120001), g.GQA_ERR_INVALID),
    (dict(scale=0.0), g.GQA_ERR_INVALID),
    (dict(scale=float("nan")), g.GQA_ERR_INVALID),
    (dict(hq=4), g.GQA_ERR_UNSUPPORTED),
    (dict(d=128), g.GQA_ERR_UNSUPPORTED),
    (dict(), g.GQA_ERR_WORKSPACE),                         # workspace required, none given
    (dict(ws=FAKE, ws_bytes=1024), g.GQA_ERR_WORKSPACE),   # too small
])
def test_prefill_rejects_before_launch(kw, status):
    assert _prefill(**kw) == status


def test_profile_stop_without_start_is_invalid():
    ms, n = ctypes.c_double(), ctypes.c_int32()
    assert g.lib().gqa_profile_stop(ctypes.byref(ms), ctypes.byref(n)) == g.GQA_ERR_INVALID
