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


def _expected_prefill_workspace(nq, q_pos0, hq=6):
    """The key-split rule restated: q-blocks of 256 packed rows, each cut into the smallest power of two
    (at most 8) of key ranges that gives at least 512 pieces, never more than its shortest q-block has
    64-key tiles; each piece of a split q-block leaves a 256-row fp32 partial (acc, m, l).  Workloads
    whose 256-row schedule has fewer than 256 pieces run 128-row q-blocks, whose partials never need
    more room (see test_small_workload_schedule_fits_the_workspace)."""
    rows = nq * hq
    nqb = -(-rows // 256)
    tiles = [(q_pos0 + min((b + 1) * 256 - 1, rows - 1) // 6 + 64) // 64 for b in range(nqb)]
    split = 1
    while split < 8 and nqb * split < 512 and split * 2 <= min(tiles):
        split *= 2
    return 0 if split == 1 else nqb * split * (256 * 256 + 2 * 256) * 4


@pytest.mark.parametrize("nq,n_kv,q_pos0", [(8000, 128000, 120000), (8000, 40000, 32000), (256, 40000, 39744),
                                             (777, 2500, 1723), (7, 100, 93), (1, 64, 63), (300, 300, 0)])
def test_prefill_workspace_follows_the_key_split(nq, n_kv, q_pos0):
    assert _ws(nq, n_kv, q_pos0) == (g.GQA_OK, _expected_prefill_workspace(nq, q_pos0))


def _schedule(nq, q_pos0, rows, hq=6):
    nr = nq * hq
    nqb = -(-nr // rows)
    tiles = [(q_pos0 + min((b + 1) * rows - 1, nr - 1) // 6 + 64) // 64 for b in range(nqb)]
    split = 1
    while split < 8 and nqb * split < 512 and split * 2 <= min(tiles):
        split *= 2
    return nqb, split


@pytest.mark.parametrize("nq,q_pos0", [(256, 768), (100, 100), (100, 1000), (40, 40), (43, 64), (1300, 3000),
                                       (777, 1723), (256, 39744), (1, 0), (7, 93), (300, 0)])
def test_small_workload_schedule_fits_the_workspace(nq, q_pos0):
    """Where the fp16 kernel takes 128-row q-blocks (the 256-row schedule has fewer than 256 pieces), the
    partials of its pieces (128 x 256 + 2 x 128 floats each) fit the workspace the query reports."""
    nqb, split = _schedule(nq, q_pos0, 256)
    if nqb * split >= 256:
        pytest.skip("256-row q-blocks")
    nqb2, split2 = _schedule(nq, q_pos0, 128)
    need = 0 if split2 == 1 else nqb2 * split2 * (128 * 256 + 2 * 128) * 4
    assert _ws(nq, nq + q_pos0, q_pos0) == (g.GQA_OK, _expected_prefill_workspace(nq, q_pos0))
    assert need <= _expected_prefill_workspace(nq, q_pos0)


def test_prefill_workspace_query():
    st, n = _ws(8000, 128000, 120000)
    assert st == g.GQA_OK and n == 752 * 264192  # 188 q-blocks x 4 key ranges
    assert _ws(1, 1, 0) == (g.GQA_OK, 0)
    assert _ws(0, 10, 0)[0] == g.GQA_ERR_INVALID
    assert _ws(10, 10, 1)[0] == g.GQA_ERR_INVALID        # q_pos0 + nq > n_kv
    assert _ws(10, 10, 0, hq=8)[0] == g.GQA_ERR_UNSUPPORTED
    assert _ws(10, 10, 0, d=128)[0] == g.GQA_ERR_UNSUPPORTED
    assert _ws(10, 10, 0, hq=12, hkv=2)[0] == g.GQA_ERR_UNSUPPORTED
    assert g.lib().gqa_prefill_causal_workspace_size(1, 1, 0, 6, 1, 256, None) == g.GQA_ERR_INVALID


def test_prefill_sizes_stop_at_the_32_bit_buffer_range():
    """Every tensor is reached through 32-bit byte offsets: K/V rows up to 2^32 - 1 bytes, Q/O likewise."""
    assert _ws(1, 8388607, 8388606)[0] == g.GQA_OK                     # 8388607 keys x 512 B < 2^32
    assert _ws(1, 8388608, 8388607)[0] == g.GQA_ERR_UNSUPPORTED        # 2^32 bytes of K
    assert _ws(1398101, 1398101, 0)[0] == g.GQA_OK                     # 1398101 x 6 rows x 512 B < 2^32
    assert _ws(1398102, 1398102, 0)[0] == g.GQA_ERR_UNSUPPORTED


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


def _paged(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, n_table=257, n_pages=512, page_size=16, offs=FAKE, ids=FAKE,
             n_ids=1000, qbr=64, kbt=4, nq=4096, q_pos0=1, live_len=4097, hq=6, hkv=1, d=256, scale=0.0625, o=FAKE,
             ws=None, ws_bytes=0)
    a.update(kw)
    return g.lib().gqa_prefill_paged_sparse(a["q"], a["kc"], a["vc"], a["pt"], a["n_table"], a["n_pages"],
                                            a["page_size"], a["offs"], a["ids"], a["n_ids"], a["qbr"], a["kbt"],
                                            a["nq"], a["q_pos0"], a["live_len"], a["hq"], a["hkv"], a["d"],
                                            a["scale"], a["o"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), g.GQA_ERR_INVALID),
    (dict(pt=None), g.GQA_ERR_INVALID),
    (dict(ids=None), g.GQA_ERR_INVALID),
    (dict(live_len=4096), g.GQA_ERR_INVALID),       # q_pos0 + nq > live_len
    (dict(live_len=257 * 16 + 1), g.GQA_ERR_INVALID),  # live tokens beyond the table
    (dict(n_pages=0), g.GQA_ERR_INVALID),
    (dict(page_size=30), g.GQA_ERR_UNSUPPORTED),    # pages must hold whole 4-token blocks
    (dict(page_size=8192, n_pages=2), g.GQA_ERR_UNSUPPORTED),
    (dict(page_size=784, n_table=6, n_pages=12), g.GQA_ERR_WORKSPACE),  # the page-784 geometry is accepted
    (dict(page_size=784, n_table=5, n_pages=12), g.GQA_ERR_INVALID),    # 5 pages of 784 < live_len
    (dict(kbt=8), g.GQA_ERR_UNSUPPORTED),
    (dict(qbr=128), g.GQA_ERR_UNSUPPORTED),
    (dict(hq=8), g.GQA_ERR_UNSUPPORTED),
    (dict(), g.GQA_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=64), g.GQA_ERR_WORKSPACE),
    # 2^20 pages of 4096 tokens: logical positions past the int32 range
    (dict(n_table=1 << 20, page_size=4096, n_pages=1), g.GQA_ERR_UNSUPPORTED),
    (dict(n_table=(1 << 31) // 4096, page_size=4096, n_pages=1), g.GQA_ERR_UNSUPPORTED),  # exactly 2^31 tokens
    (dict(n_table=(1 << 31) // 4096 - 1, page_size=4096, n_pages=1), g.GQA_ERR_WORKSPACE),  # just below: accepted
    # a workspace past the 32-bit range (ids, then the fixed partial slots)
    (dict(n_ids=525_000_000), g.GQA_ERR_UNSUPPORTED),
])
def test_paged_rejects_before_launch(kw, status):
    assert _paged(**kw) == status


@pytest.mark.parametrize("nq,n_ids", [(4096, 1000), (4096, 64 * 128), (4096, 64 * 512), (4096, 64 * 32),
                                       (128, 6048), (64, 1), (200000, 3125 * 512)])
def test_paged_workspace_follows_the_layout(nq, n_ids):
    """Restated: a 16-byte header, four int32 per 64-token query block (rounded up to 16 bytes), 8 bytes
    per id (rounded up to 256 bytes), then the partial slots: two per workgroup of the 168 teams of three
    that share the work, one fp32 partial of 128 rows (132096 bytes) each."""
    nqb = -(-nq // 64)
    entries = -(-(16 + 16 * nqb) // 16) * 16
    part = -(-(entries + 8 * max(n_ids, 1)) // 256) * 256
    n = ctypes.c_size_t()
    assert g.lib().gqa_prefill_paged_sparse_workspace_size(nq, n_ids, 64, 4, 6, 1, 256, ctypes.byref(n)) == g.GQA_OK
    assert n.value == part + 1008 * (128 * 256 + 2 * 128) * 4


def test_paged_workspace_stops_at_the_32_bit_range():
    """The workspace is addressed with 32-bit byte offsets: a layout past 2^32 - 1 bytes is refused."""
    n = ctypes.c_size_t()
    # 525,000,000 ids (4.2 GB) fit the id check, but the partial slots behind them do not
    assert g.lib().gqa_prefill_paged_sparse_workspace_size(4096, 525_000_000, 64, 4, 6, 1, 256,
                                                           ctypes.byref(n)) == g.GQA_ERR_UNSUPPORTED
    assert g.lib().gqa_prefill_paged_sparse_workspace_size(4096, 500_000_000, 64, 4, 6, 1, 256,
                                                           ctypes.byref(n)) == g.GQA_OK
    assert 4.0e9 < n.value < 2 ** 32


def test_paged_workspace_query():
    n = ctypes.c_size_t()
    assert g.lib().gqa_prefill_paged_sparse_workspace_size(4096, 1000, 64, 4, 6, 1, 256, ctypes.byref(n)) == 0
    assert n.value >= 1000 * 8
    assert g.lib().gqa_prefill_paged_sparse_workspace_size(0, 1000, 64, 4, 6, 1, 256, ctypes.byref(n)) == \
        g.GQA_ERR_INVALID


def _verify(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.01, vs=0.01, o=FAKE, nq=8, n_kv=261888, hq=6, hkv=1, d=256, scale=0.0625,
             ws=None, ws_bytes=0)
    a.update(kw)
    return g.lib().gqa_verify_fp8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["nq"], a["n_kv"], a["hq"],
                                    a["hkv"], a["d"], a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), g.GQA_ERR_INVALID),
    (dict(ks=0.0), g.GQA_ERR_INVALID),
    (dict(vs=float("inf")), g.GQA_ERR_INVALID),
    (dict(nq=0), g.GQA_ERR_INVALID),
    (dict(nq=10, n_kv=5), g.GQA_ERR_INVALID),
    (dict(nq=9), g.GQA_ERR_UNSUPPORTED),             # 54 packed rows > 48
    (dict(n_kv=262145), g.GQA_ERR_UNSUPPORTED),      # past the 262144 capability
    (dict(d=128), g.GQA_ERR_UNSUPPORTED),
    (dict(), g.GQA_ERR_WORKSPACE),
])
def test_verify_rejects_before_launch(kw, status):
    assert _verify(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), g.GQA_ERR_INVALID),
    (dict(o=None), g.GQA_ERR_INVALID),
    (dict(ks=0.0), g.GQA_ERR_INVALID),
    (dict(nq=0), g.GQA_ERR_INVALID),
    (dict(nq=10, n_kv=5), g.GQA_ERR_INVALID),
    (dict(nq=9), g.GQA_ERR_UNSUPPORTED),
    (dict(n_kv=262145), g.GQA_ERR_UNSUPPORTED),
    (dict(hq=8), g.GQA_ERR_UNSUPPORTED),
])
def test_verify_noalloc_rejects_before_launch(kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.01, vs=0.01, o=FAKE, nq=8, n_kv=261888, hq=6, hkv=1, d=256, scale=0.0625)
    a.update(kw)
    assert g.lib().gqa_verify_fp8kv_noalloc(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["nq"], a["n_kv"],
                                            a["hq"], a["hkv"], a["d"], a["scale"], None) == status


def test_verify_noalloc_scratch_holds_every_valid_call():
    """The fixed scratch (512 slots of 64 rows, 33,816,576 bytes) covers the workspace of every accepted
    verifier call; the largest is nq = 8 at the 262144-token capability."""
    n = ctypes.c_size_t()
    worst = 0
    for nq in range(1, 9):
        for n_kv in (nq, 4096, 100000, 261888, 262144):
            assert g.lib().gqa_verify_fp8kv_workspace_size(nq, n_kv, 6, 1, 256, ctypes.byref(n)) == g.GQA_OK
            worst = max(worst, n.value)
    assert worst == 512 * (64 * 256 + 2 * 64) * 4 == 33816576


def test_paged_dropped_rejects_null():
    n = ctypes.c_int32()
    assert g.lib().gqa_prefill_paged_sparse_dropped(None, ctypes.byref(n), None) == g.GQA_ERR_INVALID


def test_profile_clock_before_any_session_is_zero():
    mhz = ctypes.c_double(-1.0)
    assert g.lib().gqa_profile_clock_mhz(ctypes.byref(mhz)) == g.GQA_OK
    assert mhz.value == 0.0
    assert g.lib().gqa_profile_clock_mhz(None) == g.GQA_ERR_INVALID


def _varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, cu_q=FAKE, cu_kv=FAKE, batch=3, total_q=100, total_kv=300,
             hq=6, hkv=1, d=256, scale=0.0625, ws=None, ws_bytes=0)
    a.update(kw)
    return g.lib().gqa_prefill_causal_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"], a["cu_kv"],
                                             a["batch"], a["total_q"], a["total_kv"], a["hq"], a["hkv"], a["d"],
                                             a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), g.GQA_ERR_INVALID),
    (dict(cu_q=None), g.GQA_ERR_INVALID),
    (dict(cu_kv=None), g.GQA_ERR_INVALID),
    (dict(batch=0), g.GQA_ERR_INVALID),
    (dict(total_q=-1), g.GQA_ERR_INVALID),
    (dict(scale=float("nan")), g.GQA_ERR_INVALID),
    (dict(hq=8), g.GQA_ERR_UNSUPPORTED),
    (dict(batch=(1 << 20) + 1), g.GQA_ERR_UNSUPPORTED),
    (dict(), g.GQA_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=16), g.GQA_ERR_WORKSPACE),
])
def test_varlen_rejects_before_launch(kw, status):
    assert _varlen(**kw) == status


@pytest.mark.parametrize("batch,total_q", [(8, 27606), (8, 40000), (1, 300), (3, 1), (64, 64)])
def test_varlen_workspace_follows_the_schedule(batch, total_q):
    """Restated: at most cap = ceil(6 total_q / 256) + batch q-blocks, each cut into the smallest power of
    two (at most 8) of key ranges giving 1024 pieces; a 16-byte header and 8 int32 per q-block, rounded
    up to 256 bytes, then one 264192-byte partial per piece when the split is above 1."""
    cap = -(-6 * total_q // 256) + batch
    split = 1
    while split < 8 and cap * split < 1024:
        split *= 2
    head = -(-(16 + cap * 8 * 4) // 256) * 256
    n = ctypes.c_size_t()
    assert g.lib().gqa_prefill_causal_varlen_workspace_size(batch, total_q, 6, 1, 256, ctypes.byref(n)) == g.GQA_OK
    assert n.value == head + (cap * split * 264192 if split > 1 else 0)


@pytest.mark.parametrize("nq,n_kv", [(1, 261888), (8, 262144), (4, 4096), (2, 100), (1, 1)])
def test_verify_workspace_follows_the_schedule(nq, n_kv):
    """Restated: one 64-row fp32 partial (66048 bytes) per workgroup, with ceil(n_kv / 32) tiles spread
    at 8 or more per workgroup over between 1 and 512 workgroups."""
    grid = min(512, max(1, -(-n_kv // 32) // 8))
    n = ctypes.c_size_t()
    assert g.lib().gqa_verify_fp8kv_workspace_size(nq, n_kv, 6, 1, 256, ctypes.byref(n)) == g.GQA_OK
    assert n.value == grid * (64 * 256 + 2 * 64) * 4


def test_varlen_workspace_query():
    n = ctypes.c_size_t()
    assert g.lib().gqa_prefill_causal_varlen_workspace_size(8, 40000, 6, 1, 256, ctypes.byref(n)) == g.GQA_OK
    assert n.value > 0
    assert g.lib().gqa_prefill_causal_varlen_workspace_size(0, 10, 6, 1, 256, ctypes.byref(n)) == g.GQA_ERR_INVALID
    assert g.lib().gqa_prefill_causal_varlen_skipped(None, ctypes.byref(ctypes.c_int32()), None) == g.GQA_ERR_INVALID


def _e4m3(**kw):
    a = dict(q=FAKE, qs=0.01, k=FAKE, ks=0.01, v=FAKE, vs=0.01, o=FAKE, nq=8000, n_kv=128000, q_pos0=120000, hq=6,
             hkv=1, d=256, scale=0.0625, ws=None, ws_bytes=0)
    a.update(kw)
    return g.lib().gqa_prefill_causal_e4m3(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["nq"],
                                           a["n_kv"], a["q_pos0"], a["hq"], a["hkv"], a["d"], a["scale"], a["ws"],
                                           a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), g.GQA_ERR_INVALID),
    (dict(v=None), g.GQA_ERR_INVALID),
    (dict(qs=0.0), g.GQA_ERR_INVALID),
    (dict(ks=float("nan")), g.GQA_ERR_INVALID),
    (dict(vs=-1.0), g.GQA_ERR_INVALID),
    (dict(q_pos0=120001), g.GQA_ERR_INVALID),
    (dict(hq=8), g.GQA_ERR_UNSUPPORTED),
    (dict(d=128), g.GQA_ERR_UNSUPPORTED),
    (dict(), g.GQA_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=1024), g.GQA_ERR_WORKSPACE),
])
def test_e4m3_prefill_rejects_before_launch(kw, status):
    assert _e4m3(**kw) == status


def test_binding_rejects_host_workspace():
    """A workspace in host memory is refused before any call reaches the library."""
    import torch

    with pytest.raises(ValueError, match="device memory"):
        g._workspace(1024, torch.device("cpu"), torch.empty(1024, dtype=torch.uint8))
    assert g._workspace(0, torch.device("cpu"), None) == (None, 0)


def test_binding_checks_shapes_before_pointers_leave():
    """The kernels size buffers from the call's arguments: a mismatched output or cache shape is refused."""
    import torch

    t = torch.empty((4, 6, 256), dtype=torch.float16)
    with pytest.raises(ValueError, match="device memory"):  # checked in order: placement first
        g._dev(t, torch.float16, "o", (4, 6, 256))
    if not torch.cuda.is_available():
        return
    d = t.cuda()
    with pytest.raises(ValueError, match="shape"):
        g._dev(d, torch.float16, "o", (5, 6, 256))
