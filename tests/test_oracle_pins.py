"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages print no worked input/output example, so the oracle is pinned by
closed forms, library routines that compute the same definition, brute force
on tiny inputs, and invariants that the definition implies.  Each pin names the
mistake it guards against.  ``test_planted_mistakes_are_caught`` plants those
mistakes in the oracle (on the CPU) and checks that a pin fails for each.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import attention as oatt
import workloads

SCALE = 1.0 / 16.0


def _rand(shape, seed, dtype=np.float64):
    return np.random.default_rng(seed).standard_normal(shape).astype(dtype)


# ---------------------------------------------------------------- E4M3 format
def test_e4m3_spec_values():
    """Code points fixed by the OCP E4M3 definition (bias 7, no inf, S.1111.111 = NaN)."""
    t = oracle.e4m3_table()
    assert t[0x00] == 0.0 and math.copysign(1, t[0x80]) == -1.0
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0x7E] == 448.0                # largest finite
    assert t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254


def test_e4m3_matches_torch_float8():
    """All 256 codes agree with torch's float8_e4m3fn decoding (library routine)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes.numpy())
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_e4m3_values_exact_in_fp16():
    """Every finite E4M3 value is exactly representable in fp16 (decode -> fp16 MFMA is exact)."""
    t = oracle.e4m3_table()
    f = t[np.isfinite(t)]
    assert np.array_equal(f.astype(np.float16).astype(np.float64), f)


def test_generator_quantiser_is_nearest():
    """The generator's float8 cast picks the nearest E4M3 value (brute force over all codes)."""
    t = oracle.e4m3_table()
    fin = np.isfinite(t)
    vals = t[fin]
    x = _rand((2000,), 3, np.float32) * np.float32(100.0)
    codes = workloads._to_e4m3(x, np.float32(1.0))
    dec = oracle.e4m3_decode(codes)
    dist = np.abs(x.astype(np.float64)[:, None] - vals[None, :])
    best = dist.min(axis=1)
    assert np.all(np.abs(x - dec) <= best + 1e-12)


# ----------------------------------------------------------- attention core pins
def test_single_visible_key_returns_its_value():
    """A row that sees only key 0 returns V[0] exactly (guards the mask boundary)."""
    q = _rand((3, 6, 8), 1); k = _rand((3, 1, 8), 2); v = _rand((3, 1, 8), 3)
    o, lse = oracle.prefill_causal(q, k, v, 0, SCALE)
    assert np.array_equal(o[0], np.repeat(v[0], 6, axis=0))
    # lse of a single key is its own score
    np.testing.assert_allclose(lse[0], SCALE * (q[0] @ k[0, 0]), rtol=0, atol=1e-14)


def test_constant_values_give_constant_output():
    """V rows all equal c gives O = c for every row (normalisation by the weight sum)."""
    q = _rand((7, 6, 16), 4); k = _rand((20, 1, 16), 5)
    c = _rand((16,), 6)
    v = np.broadcast_to(c, (20, 1, 16)).copy()
    o, _ = oracle.prefill_causal(q, k, v, 13, SCALE)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


def test_zero_keys_give_prefix_mean():
    """K = 0 makes all scores equal, so row r returns the mean of V[0..pos_r] (causal extent)."""
    nq, L, q_pos0 = 9, 30, 21
    q = _rand((nq, 6, 8), 7); k = np.zeros((L, 1, 8)); v = _rand((L, 1, 8), 8)
    o, lse = oracle.prefill_causal(q, k, v, q_pos0, SCALE)
    for r in range(nq):
        p = q_pos0 + r
        np.testing.assert_allclose(o[r], np.repeat(v[:p + 1, 0].mean(axis=0)[None], 6, axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[r], np.log(p + 1), atol=1e-13)


def test_two_keys_logistic_closed_form():
    """With two visible keys O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1 (sign and scale of scores)."""
    d = 32
    q = _rand((1, 6, d), 9); k = _rand((2, 1, d), 10); v = _rand((2, 1, d), 11)
    o, lse = oracle.prefill_causal(q, k, v, 1, SCALE)
    for h in range(6):
        s0 = SCALE * float(np.dot(q[0, h], k[0, 0]))
        s1 = SCALE * float(np.dot(q[0, h], k[1, 0]))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(o[0, h], w0 * v[0, 0] + w1 * v[1, 0], atol=1e-14)
        np.testing.assert_allclose(lse[0, h], max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), atol=1e-14)


def _torch_sdpa(q, k, v, q_pos0, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, GQA by enable_gqa."""
    nq, L = q.shape[0], k.shape[0]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    if q_pos0 == 0 and nq == L:
        out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
    else:
        assert q_pos0 + nq == L
        kt = kt.repeat_interleave(q.shape[1] // k.shape[1], dim=1)
        vt = vt.repeat_interleave(q.shape[1] // k.shape[1], dim=1)
        out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal_lower_right(nq, L), scale=scale)
    return out[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("hq,hkv", [(6, 1), (12, 2), (4, 4)])
def test_matches_torch_sdpa_square_causal(hq, hkv):
    """Square causal case equals torch SDPA with is_causal=True and enable_gqa (head mapping, scale)."""
    L, d = 37, 24
    q = _rand((L, hq, d), 12); k = _rand((L, hkv, d), 13); v = _rand((L, hkv, d), 14)
    o, _ = oracle.prefill_causal(q, k, v, 0, SCALE)
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, 0, SCALE), atol=1e-13, rtol=0)


def test_matches_torch_sdpa_lower_right():
    """Queries at the last positions equal torch SDPA with the lower-right causal bias."""
    nq, L, d = 11, 53, 16
    q = _rand((nq, 6, d), 15); k = _rand((L, 1, d), 16); v = _rand((L, 1, d), 17)
    o, _ = oracle.prefill_causal(q, k, v, L - nq, SCALE)
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, L - nq, SCALE), atol=1e-13, rtol=0)


def _brute(q, k, v, vis_fn, scale, group):
    """Pure-Python attention: explicit loops, math.exp, math.fsum (no numpy)."""
    nq, hq, d = q.shape
    out = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    for r in range(nq):
        for h in range(hq):
            g = h // group
            keys = [j for j in range(k.shape[0]) if vis_fn(r, j)]
            if not keys:
                continue
            s = [scale * math.fsum(float(q[r, h, i]) * float(k[j, g, i]) for i in range(d)) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = math.fsum(w)
            for i in range(d):
                out[r][h][i] = math.fsum(wj * float(v[j, g, i]) for wj, j in zip(w, keys)) / den
    return np.array(out)


def test_brute_force_tiny_causal():
    nq, L, d, q_pos0 = 5, 9, 4, 4
    q = _rand((nq, 6, d), 18); k = _rand((L, 1, d), 19); v = _rand((L, 1, d), 20)
    o, _ = oracle.prefill_causal(q, k, v, q_pos0, SCALE)
    ref = _brute(q, k, v, lambda r, j: j <= q_pos0 + r, SCALE, 6)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_rows_subset_matches_full():
    """Evaluating a sampled subset of rows gives the same rows as the full evaluation."""
    q = _rand((40, 6, 8), 21); k = _rand((70, 1, 8), 22); v = _rand((70, 1, 8), 23)
    o, lse = oracle.prefill_causal(q, k, v, 30, SCALE)
    rows = np.array([39, 0, 17, 5])
    o2, lse2 = oracle.prefill_causal(q, k, v, 30, SCALE, rows=rows)
    np.testing.assert_allclose(o2, o[rows], atol=1e-15, rtol=0)
    np.testing.assert_allclose(lse2, lse[rows], atol=1e-15, rtol=0)


# ------------------------------------------------------------------- invariants
def test_causality_future_keys_do_not_matter():
    """Changing K/V at positions after a row's position leaves that row bit-identical."""
    nq, L, q_pos0 = 6, 20, 10
    q = _rand((nq, 6, 8), 24); k = _rand((L, 1, 8), 25); v = _rand((L, 1, 8), 26)
    for r in range(nq):
        p = q_pos0 + r
        k2, v2 = k.copy(), v.copy()
        k2[p + 1:] += 5.0
        v2[p + 1:] -= 3.0
        o1, _ = oracle.prefill_causal(q, k, v, q_pos0, SCALE, rows=[r])
        o2, _ = oracle.prefill_causal(q, k2, v2, q_pos0, SCALE, rows=[r])
        assert np.array_equal(o2[0], o1[0])


def test_key_shift_invariance():
    """Adding one vector to every key shifts each row's scores by a constant: O unchanged."""
    q = _rand((8, 6, 16), 27); k = _rand((24, 1, 16), 28); v = _rand((24, 1, 16), 29)
    c = _rand((16,), 30)
    o, _ = oracle.prefill_causal(q, k, v, 16, SCALE)
    o2, _ = oracle.prefill_causal(q, k + c[None, None, :], v, 16, SCALE)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)


def test_head_permutation_equivariance():
    """Permuting query heads inside one K/V group permutes the output heads."""
    q = _rand((8, 6, 16), 31); k = _rand((24, 1, 16), 32); v = _rand((24, 1, 16), 33)
    perm = np.array([3, 0, 5, 1, 4, 2])
    o, _ = oracle.prefill_causal(q, k, v, 16, SCALE)
    o2, _ = oracle.prefill_causal(q[:, perm], k, v, 16, SCALE)
    assert np.array_equal(o2, o[:, perm])


def test_lse_merge_of_a_partition_is_exact():
    """Merging (O, lse) of two disjoint key subsets by log-sum-exp equals the unsplit result."""
    n, L, d = 10, 40, 16
    q = _rand((n, d), 34); k = _rand((L, d), 35); v = _rand((L, d), 36)
    vis = np.ones((n, L), dtype=bool)
    o, lse = oracle.attend(q, k, v, vis, SCALE)
    cut = 17
    oa, la = oracle.attend(q, k[:cut], v[:cut], vis[:, :cut], SCALE)
    ob, lb = oracle.attend(q, k[cut:], v[cut:], vis[:, cut:], SCALE)
    mm = np.maximum(la, lb)
    wa, wb = np.exp(la - mm), np.exp(lb - mm)
    om = (wa[:, None] * oa + wb[:, None] * ob) / (wa + wb)[:, None]
    np.testing.assert_allclose(om, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(mm + np.log(wa + wb), lse, atol=1e-13, rtol=0)


def test_empty_visible_set_is_zero():
    q = _rand((2, 4), 37); k = _rand((3, 4), 38); v = _rand((3, 4), 39)
    vis = np.array([[False, False, False], [True, False, False]])
    o, lse = oracle.attend(q, k, v, vis, SCALE)
    assert np.array_equal(o[0], np.zeros(4)) and lse[0] == -np.inf
    assert np.array_equal(o[1], v[0])


def test_visible_pair_count_matches_configs():
    """Visible pairs: 8000*KV - 31,996,000 for Q=8000 at the last positions."""
    for kv in (40000, 128000):
        assert oracle.visible_pairs_causal(8000, kv, kv - 8000) == 8000 * kv - 31_996_000
    assert oracle.visible_pairs_causal(256, 1024, 768) == 229_504


# --------------------------------------------------------------- paged / sparse
def _paged_small(tail, seed, **kw):
    return workloads.paged_sparse_inputs(select_tokens=16, tail=tail, seed=seed, nq=150, n_pages=24, d=16, **kw)


def _run_paged(x, **over):
    args = dict(q=x.q, k_cache=x.k_cache, v_cache=x.v_cache, page_table=x.page_table, page_size=x.page_size,
                qblock_offsets=x.qblock_offsets, kv_block_ids=x.kv_block_ids, qblock_rows=x.qblock_rows,
                kv_block_tokens=x.kv_block_tokens, q_pos0=x.q_pos0, live_len=x.live_len, scale=x.scale)
    args.update(over)
    return oracle.prefill_paged_sparse(**args)


@pytest.mark.parametrize("tail", [0, 1, 2, 3])
def test_paged_saturated_equals_dense_causal(tail):
    """Selecting every block up to the diagonal reproduces dense causal attention over the positions."""
    x = _paged_small(tail, 40 + tail, saturate=True)
    o, lse = _run_paged(x)
    toks = np.arange(x.live_len)
    kc = oatt.gather_paged(x.k_cache, x.page_table, 16, toks)
    vc = oatt.gather_paged(x.v_cache, x.page_table, 16, toks)
    od, lsed = oracle.prefill_causal(x.q, kc, vc, x.q_pos0, x.scale)
    np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lsed, atol=1e-12, rtol=0)


def test_paged_table_permutation_is_transparent():
    """The same logical cache behind the identity table and a permuted table gives identical output."""
    x = _paged_small(2, 44)
    o, _ = _run_paged(x)
    n_table = x.page_table.size
    toks = np.arange(n_table * 16)
    k_log = oatt.gather_paged(x.k_cache, x.page_table, 16, toks).reshape(n_table, 16, 1, -1)
    v_log = oatt.gather_paged(x.v_cache, x.page_table, 16, toks).reshape(n_table, 16, 1, -1)
    o2, _ = _run_paged(x, k_cache=k_log, v_cache=v_log, page_table=np.arange(n_table, dtype=np.int32))
    assert np.array_equal(o, o2)


def test_paged_block_order_is_irrelevant():
    x = _paged_small(1, 45)
    o, _ = _run_paged(x)
    ids = x.kv_block_ids.copy()
    for b in range(x.qblock_offsets.size - 1):
        s, e = x.qblock_offsets[b], x.qblock_offsets[b + 1]
        ids[s:e] = np.sort(ids[s:e])[::-1]
    o2, _ = _run_paged(x, kv_block_ids=ids)
    assert np.array_equal(o, o2)


def test_paged_stale_poison_is_clamped():
    """NaN in every slot that holds no live token changes nothing (clamp to the live length)."""
    x = _paged_small(3, 46)
    xp = _paged_small(3, 46, poison_stale=True)
    assert np.isnan(xp.k_cache).any()
    o, _ = _run_paged(x)
    o2, _ = _run_paged(xp)
    assert np.isfinite(o2).all()
    assert np.array_equal(o, o2)


def test_paged_brute_force_tiny():
    """Tiny paged case against pure-Python attention with the visibility rule spelled out."""
    x = workloads.paged_sparse_inputs(select_tokens=8, tail=2, seed=47, nq=10, n_pages=4, d=4)
    x.qblock_rows = 4
    # rebuild a CSR for 4-row blocks by hand: block b selects its own diagonal block and block 0
    nblk = 3
    ids, offs = [], [0]
    for b in range(nblk):
        last = x.q_pos0 + min(10, 4 * b + 4) - 1
        sel = sorted({last // 4, 0})
        ids += sel
        offs.append(len(ids))
    x.kv_block_ids = np.array(ids, dtype=np.int32)
    x.qblock_offsets = np.array(offs, dtype=np.int32)
    o, _ = _run_paged(x)
    L = x.live_len
    toks = np.arange(L)
    kc = oatt.gather_paged(x.k_cache, x.page_table, 16, toks)
    vc = oatt.gather_paged(x.v_cache, x.page_table, 16, toks)

    def vis(r, j):
        b = r // 4
        blocks = ids[offs[b]:offs[b + 1]]
        return (j // 4) in blocks and j <= x.q_pos0 + r and j < L

    ref = _brute(x.q.astype(np.float64), kc.astype(np.float64), vc.astype(np.float64), vis, x.scale, 6)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_paged_empty_row_is_zero():
    """A row whose selection holds no visible token outputs exactly zero."""
    x = workloads.paged_sparse_inputs(select_tokens=8, tail=0, seed=48, nq=64, n_pages=8, d=8)
    x.kv_block_ids = np.array([15], dtype=np.int32)  # only the diagonal block (positions 60..63)
    x.qblock_offsets = np.array([0, 1], dtype=np.int32)
    o, lse = _run_paged(x)
    assert np.array_equal(o[:60], np.zeros_like(o[:60]))
    assert np.all(lse[:60] == -np.inf)
    assert np.isfinite(o[60:]).all() and np.all(np.isfinite(lse[60:]))


# ------------------------------------------------------------------ FP8 verifier
def test_verify_equals_causal_on_decoded_values():
    """The verifier is causal attention of the last rows over decode(byte) * scale."""
    x = workloads.verify_inputs(4, 300, seed=49, d=32)
    o, lse = oracle.verify_fp8kv(x.q, x.k_bytes, x.v_bytes, x.k_scale, x.v_scale, x.scale)
    kd = torch.from_numpy(x.k_bytes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * x.k_scale
    vd = torch.from_numpy(x.v_bytes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * x.v_scale
    ref = _torch_sdpa(x.q.astype(np.float64), kd, vd, 300 - 4, x.scale)
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)


def test_verify_generator_scale_is_amax_over_448():
    x = workloads.verify_inputs(2, 500, seed=50, d=16)
    dec = oracle.e4m3_decode(x.k_bytes)
    assert np.abs(dec).max() == 448.0
    assert x.k_scale > 0 and x.v_scale > 0


# -------------------------------------------------------- E4M3 causal prefill
def _torch_dec(codes, scale):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * np.float64(np.float32(scale))


def test_prefill_e4m3_equals_sdpa_on_torch_decoded_values():
    """The E4M3 prefill is causal attention of decode(byte) * scale for Q, K and V
    (torch's float8 decoding and torch SDPA as the library routines)."""
    x = workloads.e4m3_prefill_inputs(24, 70, seed=51, d=32)
    o, lse = oracle.prefill_causal_e4m3(x.q_bytes, x.q_scale, x.k_bytes, x.k_scale, x.v_bytes, x.v_scale,
                                        x.q_pos0, x.scale)
    ref = _torch_sdpa(_torch_dec(x.q_bytes, x.q_scale), _torch_dec(x.k_bytes, x.k_scale),
                      _torch_dec(x.v_bytes, x.v_scale), x.q_pos0, x.scale)
    np.testing.assert_allclose(o, ref, atol=1e-13, rtol=0)


def test_prefill_e4m3_brute_force_tiny():
    """Pure-Python attention over the spec decoding of the codes."""
    x = workloads.e4m3_prefill_inputs(4, 7, seed=52, d=4)
    o, _ = oracle.prefill_causal_e4m3(x.q_bytes, x.q_scale, x.k_bytes, x.k_scale, x.v_bytes, x.v_scale,
                                      x.q_pos0, x.scale)
    t = oracle.e4m3_table()
    dec = lambda b, sc: np.vectorize(lambda c: float(t[c]) * float(np.float32(sc)))(b)
    ref = _brute(dec(x.q_bytes, x.q_scale), dec(x.k_bytes, x.k_scale), dec(x.v_bytes, x.v_scale),
                 lambda r, j: j <= x.q_pos0 + r, x.scale, 6)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_prefill_e4m3_scales_enter_where_the_definition_puts_them():
    """Doubling the Q scale while halving the softmax scale changes nothing; doubling
    the V scale doubles O; doubling the K scale is the same as doubling the softmax scale."""
    x = workloads.e4m3_prefill_inputs(6, 20, seed=53, d=8)
    args = (x.q_bytes, x.q_scale, x.k_bytes, x.k_scale, x.v_bytes, x.v_scale, x.q_pos0)
    o, lse = oracle.prefill_causal_e4m3(*args, x.scale)
    o2, lse2 = oracle.prefill_causal_e4m3(x.q_bytes, 2 * x.q_scale, *args[2:], x.scale / 2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    o3, _ = oracle.prefill_causal_e4m3(*args[:5], 2 * x.v_scale, x.q_pos0, x.scale)
    assert np.array_equal(o3, 2 * o)
    o4, _ = oracle.prefill_causal_e4m3(x.q_bytes, x.q_scale, x.k_bytes, 2 * x.k_scale, *args[4:], x.scale)
    o5, _ = oracle.prefill_causal_e4m3(*args, 2 * x.scale)
    assert np.array_equal(o4, o5)


def test_e4m3_prefill_generator_scales_are_amax_over_448():
    x = workloads.e4m3_prefill_inputs(5, 30, seed=54, d=16)
    for b in (x.q_bytes, x.k_bytes, x.v_bytes):
        assert np.abs(oracle.e4m3_decode(b)).max() == 448.0
    assert x.q_pos0 == 25 and min(x.q_scale, x.k_scale, x.v_scale) > 0


# ------------------------------------------------------------- varlen prefill
def _varlen_tiny():
    kv, ql = [4, 1, 0, 6, 3], [2, 1, 0, 3, 3]  # includes a one-key sequence, an empty one, nq == nkv
    x = workloads.varlen_inputs(kv, ql, seed=41, d=4)
    return x, kv, ql


def test_varlen_brute_force_tiny():
    """Each sequence is brute-forced on its own slices with its queries at its last positions."""
    x, kv, ql = _varlen_tiny()
    o, lse = oracle.prefill_causal_varlen(x.q, x.k, x.v, x.cu_q, x.cu_kv, SCALE)
    for i in range(len(kv)):
        q0, q1, k0, k1 = x.cu_q[i], x.cu_q[i + 1], x.cu_kv[i], x.cu_kv[i + 1]
        if q1 == q0:
            continue
        start = (k1 - k0) - (q1 - q0)
        ref = _brute(x.q[q0:q1], x.k[k0:k1], x.v[k0:k1], lambda r, j: j <= start + r, SCALE, 6)
        np.testing.assert_allclose(o[q0:q1], ref, atol=1e-12, rtol=0)
    assert np.isfinite(lse).all()


def test_varlen_sequences_are_independent():
    """Changing one sequence's K/V leaves every other sequence bit-identical (and its lse too)."""
    x, kv, ql = _varlen_tiny()
    o, lse = oracle.prefill_causal_varlen(x.q, x.k, x.v, x.cu_q, x.cu_kv, SCALE)
    k2, v2 = x.k.copy(), x.v.copy()
    k0, k1 = x.cu_kv[3], x.cu_kv[4]
    k2[k0:k1] += np.float16(0.5)
    v2[k0:k1] *= np.float16(-1)
    o2, lse2 = oracle.prefill_causal_varlen(x.q, k2, v2, x.cu_q, x.cu_kv, SCALE)
    other = np.ones(x.q.shape[0], dtype=bool)
    other[x.cu_q[3]:x.cu_q[4]] = False
    assert np.array_equal(o[other], o2[other]) and np.array_equal(lse[other], lse2[other])
    assert not np.array_equal(o[~other], o2[~other])


def test_varlen_lse_is_log_partition():
    """lse equals log sum_j exp(scale q.k_j) over the visible keys (closed form on one sequence)."""
    x, kv, ql = _varlen_tiny()
    _, lse = oracle.prefill_causal_varlen(x.q, x.k, x.v, x.cu_q, x.cu_kv, SCALE)
    i = 3
    q0, k0, nkv, nq = x.cu_q[i], x.cu_kv[i], kv[i], ql[i]
    for r in range(nq):
        for h in range(6):
            vis = range(nkv - nq + r + 1)
            z = math.fsum(math.exp(SCALE * math.fsum(float(x.q[q0 + r, h, t]) * float(x.k[k0 + j, 0, t])
                                                     for t in range(4))) for j in vis)
            assert abs(lse[q0 + r, h] - math.log(z)) < 1e-12


# ------------------------------------------------------------- planted mistakes
def _pin_suite():
    """Cheap pins run against a mutated oracle; returns the names that fail."""
    failed = []
    for fn in (test_single_visible_key_returns_its_value, test_zero_keys_give_prefix_mean,
               test_two_keys_logistic_closed_form, test_matches_torch_sdpa_lower_right,
               test_brute_force_tiny_causal, test_constant_values_give_constant_output):
        try:
            fn()
        except AssertionError:
            failed.append(fn.__name__)
    try:
        test_matches_torch_sdpa_square_causal(12, 2)
    except AssertionError:
        failed.append("sdpa_gqa")
    return failed


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pin_suite() == []
    real_attend = oatt.attend
    mutants = {
        "causal off by one": ("causal_visible", lambda pos, keys: keys[None, :] < pos[:, None]),
        "causal window shifted": ("causal_visible", lambda pos, keys: keys[None, :] <= pos[:, None] + 1),
        "interleaved kv heads": ("kv_head_of", lambda h, hq, hkv: h % hkv),
        "scale dropped": ("attend", lambda q, k, v, vis, scale: real_attend(q, k, v, vis, 1.0)),
        "sign flipped": ("attend", lambda q, k, v, vis, scale: real_attend(q, k, v, vis, -scale)),
        "keys swapped for values": ("attend", lambda q, k, v, vis, scale: real_attend(q, v, k, vis, scale)),
        "no normalisation": ("attend", lambda q, k, v, vis, scale: (lambda o_l: (o_l[0] * vis.sum(1, keepdims=True), o_l[1]))(real_attend(q, k, v, vis, scale))),
    }
    for name, (attr, fn) in mutants.items():
        with monkeypatch.context() as m:
            m.setattr(oatt, attr, fn)
            caught = _pin_suite()
        assert caught, f"planted mistake not caught: {name}"
