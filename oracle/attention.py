"""fp64 softmax attention, written from its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For one query row r of head h and the set V(r) of key positions it may see,

    s_j      = scale * <Q[r, h, :], K[j, g, :]>          for j in V(r)
    m        = max_j s_j
    O[r,h,:] = sum_j exp(s_j - m) V[j, g, :] / sum_j exp(s_j - m)
    lse[r,h] = m + log(sum_j exp(s_j - m))

with g = h // (Hq / Hkv), the grouped-query mapping in which consecutive query
heads share one K/V head (six query heads and one K/V head on the pages).  When
V(r) is empty the row is defined as O = 0 and lse = -inf.

The pages fix the problem, not the arithmetic of a reference: the long-prefill
page states the shape family and the FP16 accuracy envelope (Test Result:
max abs <= 1e-3, rel L2 <= 1e-2), and the block-sparse page reports an exact
kernel at about 3e-4 rel L2.  This oracle therefore evaluates the definition
above in float64 over the exact float64 images of the fp16 (or decoded E4M3)
inputs, with numpy matrix products as the only library step.  Rows are handled
in chunks purely to bound memory; nothing is reordered beyond what the
definition allows.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode

# Largest score block (rows x keys) materialised at once, in elements.
_MAX_BLOCK_ELEMS = 1 << 25


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """K/V head used by query head ``h``: consecutive groups of hq/hkv query heads share one."""
    return h // (hq // hkv)


def causal_visible(pos: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Visibility of key positions ``keys`` to query positions ``pos``.

    A query at position p sees every key at a position j <= p (a query sees
    itself and the past, never the future).
    """
    return keys[None, :] <= pos[:, None]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray, scale: float):
    """Masked softmax attention of query rows over an explicit key list.

    q: [n, D]; k, v: [m, D]; visible: bool [n, m].  Every row of ``k`` and
    ``v`` must be finite (callers pass only live keys).  Returns (o [n, D],
    lse [n]) in float64; rows with no visible key give o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    if k.shape[0] == 0 or n == 0:
        return o, lse
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    if not has.any():
        return o, lse
    w = np.exp(s[has] - m[has, None])  # masked entries: exp(-inf) = 0
    den = w.sum(axis=1)
    o[has] = (w @ v) / den[:, None]
    lse[has] = m[has] + np.log(den)
    return o, lse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def prefill_causal(q, k, v, q_pos0: int, scale: float, rows=None):
    """Dense causal GQA prefill.

    q: [nq, Hq, D]; k, v: [L, Hkv, D] (any float dtype, used as exact float64).
    Query row r sits at position q_pos0 + r and sees keys 0..q_pos0 + r.
    ``rows`` (optional, sorted or not) restricts the evaluation to those query
    rows; the result then has len(rows) rows in the given order.
    Returns (o [n, Hq, D], lse [n, Hq]).
    """
    nq, hq, d = q.shape
    L, hkv, _ = k.shape
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    o = np.zeros((n, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((n, hq), -np.inf, dtype=np.float64)
    pos_all = q_pos0 + rows
    if n == 0:
        return o, lse
    if pos_all.max() >= L or q_pos0 < 0:
        raise ValueError("query positions must lie inside the key range")
    order = np.argsort(pos_all, kind="stable")
    chunk = max(1, _MAX_BLOCK_ELEMS // max(1, L))
    for c0 in range(0, n, chunk):
        idx = order[c0:c0 + chunk]
        pos = pos_all[idx]
        m = int(pos.max()) + 1  # keys 0..max position of the chunk
        keys = np.arange(m)
        vis = causal_visible(pos, keys)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            oh, lh = attend(_as64(q[rows[idx], h, :]), _as64(k[:m, g, :]), _as64(v[:m, g, :]), vis, scale)
            o[idx, h, :] = oh
            lse[idx, h] = lh
    return o, lse


def selected_tokens(block_ids, kv_block_tokens: int, live_len: int) -> np.ndarray:
    """Token positions covered by the selected blocks, stale ones removed.

    Block b covers positions b*kv_block_tokens .. b*kv_block_tokens + kv_block_tokens - 1.
    Positions at or past the live length are padding or stale cache slots and
    never take part (clamp to the live request length).  The union is returned
    sorted; the selection is a set, so order and duplicates do not matter.
    """
    b = np.unique(np.asarray(block_ids, dtype=np.int64))
    toks = (b[:, None] * kv_block_tokens + np.arange(kv_block_tokens)[None, :]).reshape(-1)
    return np.sort(toks[toks < live_len])


def gather_paged(cache, page_table, page_size: int, tokens: np.ndarray):
    """Rows of a paged cache [n_pages, page_size, Hkv, D] at logical ``tokens``.

    Logical token j lives in physical page page_table[j // page_size], slot
    j % page_size.
    """
    pt = np.asarray(page_table, dtype=np.int64)
    pages = pt[tokens // page_size]
    slots = tokens % page_size
    return cache[pages, slots]  # [n_tokens, Hkv, D]


def prefill_causal_varlen(q, k, v, cu_q, cu_kv, scale: float):
    """Causal prefill of a batch of independent sequences packed end to end.

    Sequence i owns query rows cu_q[i] .. cu_q[i+1]-1 of q [total_q, Hq, D]
    and key rows cu_kv[i] .. cu_kv[i+1]-1 of k, v [total_kv, Hkv, D]; its
    nq_i queries are the last nq_i positions of its nkv_i keys (the causal
    convention of the dense prefill, applied per sequence; a serving engine
    batches requests this way, and the per-row lse lets a caller merge the
    result with other attention pieces).  Each sequence is exactly
    ``prefill_causal`` on its own slices, with q_pos0 = nkv_i - nq_i.
    Returns (o [total_q, Hq, D], lse [total_q, Hq]) in float64.
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    total_q, hq, d = q.shape
    o = np.zeros((total_q, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((total_q, hq), -np.inf, dtype=np.float64)
    for i in range(cu_q.size - 1):
        q0, q1, k0, k1 = cu_q[i], cu_q[i + 1], cu_kv[i], cu_kv[i + 1]
        nq, nkv = q1 - q0, k1 - k0
        if nq == 0:
            continue
        if nq > nkv:
            raise ValueError("a sequence has more queries than keys")
        oi, li = prefill_causal(q[q0:q1], k[k0:k1], v[k0:k1], int(nkv - nq), scale)
        o[q0:q1] = oi
        lse[q0:q1] = li
    return o, lse


def prefill_paged_sparse(q, k_cache, v_cache, page_table, page_size: int, qblock_offsets, kv_block_ids,
                         qblock_rows: int, kv_block_tokens: int, q_pos0: int, live_len: int, scale: float):
    """Block-sparse causal GQA prefill over a paged K/V cache.

    Query block b holds rows b*qblock_rows .. (b+1)*qblock_rows - 1 (the last
    may be short).  Its selection is kv_block_ids[qblock_offsets[b] :
    qblock_offsets[b+1]], logical block indices of kv_block_tokens tokens each.
    Row r (position q_pos0 + r) of block b sees token j iff j is in a selected
    block of b, j <= q_pos0 + r (causal within the selection), and
    j < live_len (stale slots are clamped away).
    Returns (o [nq, Hq, D], lse [nq, Hq]) in float64.
    """
    nq, hq, d = q.shape
    hkv = k_cache.shape[2]
    offs = np.asarray(qblock_offsets, dtype=np.int64)
    ids = np.asarray(kv_block_ids, dtype=np.int64)
    o = np.zeros((nq, hq, v_cache.shape[3]), dtype=np.float64)
    lse = np.full((nq, hq), -np.inf, dtype=np.float64)
    nblk = (nq + qblock_rows - 1) // qblock_rows
    for b in range(nblk):
        r0, r1 = b * qblock_rows, min(nq, (b + 1) * qblock_rows)
        toks = selected_tokens(ids[offs[b]:offs[b + 1]], kv_block_tokens, live_len)
        kb = gather_paged(k_cache, page_table, page_size, toks)
        vb = gather_paged(v_cache, page_table, page_size, toks)
        pos = q_pos0 + np.arange(r0, r1)
        vis = causal_visible(pos, toks)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            oh, lh = attend(_as64(q[r0:r1, h, :]), _as64(kb[:, g, :]), _as64(vb[:, g, :]), vis, scale)
            o[r0:r1, h, :] = oh
            lse[r0:r1, h] = lh
    return o, lse


def verify_fp8kv(q, k_bytes, v_bytes, k_scale: float, v_scale: float, scale: float, rows=None):
    """Causal verifier tail over an E4M3 K/V cache.

    k_bytes, v_bytes: uint8 [L, Hkv, D] OCP E4M3 codes; the cached values are
    decode(byte) * k_scale and decode(byte) * v_scale (one fp32 scale per
    tensor).  The nq query rows occupy the last nq positions L-nq .. L-1 and are
    causal among themselves.  Returns (o [nq, Hq, D], lse [nq, Hq]).
    """
    nq = q.shape[0]
    L = k_bytes.shape[0]
    kd = e4m3_decode(k_bytes) * np.float64(np.float32(k_scale))
    vd = e4m3_decode(v_bytes) * np.float64(np.float32(v_scale))
    return prefill_causal(q, kd, vd, L - nq, scale, rows=rows)


def prefill_causal_e4m3(q_bytes, q_scale: float, k_bytes, k_scale: float, v_bytes, v_scale: float, q_pos0: int,
                        scale: float, rows=None):
    """Dense causal GQA prefill over E4M3 inputs.

    The long-context page's E4M3 operator ("[Perf] Ship the qualified SM70
    long-context layout...", What: grouped E4M3 FP32 long-context operator)
    keeps K and V as OCP E4M3 codes with one fp32 scale per tensor.  In the
    variant whose Q K^T products run on FP8 matrix cores, Q is quantised the
    same way, so the operation is defined on the quantised queries: every
    operand is decode(byte) * its tensor's scale, and the attention is the
    dense causal prefill (``prefill_causal``) of those values, with query row
    r at position q_pos0 + r.  Returns (o [nq, Hq, D], lse [nq, Hq]).
    """
    qd = e4m3_decode(q_bytes) * np.float64(np.float32(q_scale))
    kd = e4m3_decode(k_bytes) * np.float64(np.float32(k_scale))
    vd = e4m3_decode(v_bytes) * np.float64(np.float32(v_scale))
    return prefill_causal(qd, kd, vd, q_pos0, scale, rows=rows)


def visible_pairs_causal(nq: int, n_kv: int, q_pos0: int) -> int:
    """Number of visible (query row, key) pairs of one head in causal prefill."""
    p0, p1 = q_pos0, q_pos0 + nq - 1
    assert p1 < n_kv
    return (p0 + 1 + p1 + 1) * nq // 2
