"""Seeded synthetic inputs for the causal GQA attention path.

This module draws inputs only; it holds none of the attention arithmetic and is
shared by the test suite, the benchmark and the fp64 reference.  Every array is
produced by ``numpy.random.default_rng(seed)`` (PCG64): standard normal values
drawn in float32 in the order Q, K, V and rounded to fp16 (round to nearest
even).  Shapes follow the workloads of the pages:

* causal prefill -- Hq=6 query heads sharing Hkv=1 K/V head, D=256, scale 1/16,
  Q rows at the last positions of the key range ("[Kernel][SM70] Default
  long-prefill GQA architecture", Purpose: Q=8000, KV=40000..128000 step 8000).
* paged block-sparse prefill -- 4096 query rows, page-16 cache behind a
  non-monotonic page table, 64-row query blocks selecting 4-token KV blocks,
  selections of 64 / 512 / 2048 tokens, partial tails of 0..3 tokens ("[Kernel]
  [SM70] Repair #378 on latest main", Changes and Test Result).
* FP8 verifier tail -- 2..8 query rows at the end of a 261888-token context with
  K/V stored as OCP E4M3 codes and one fp32 scale per tensor ("[Perf] Ship the
  qualified SM70 long-context layout...", Changes and Measurement).  The E4M3
  codes are produced with torch's float8_e4m3fn cast (round to nearest even)
  of value/scale with scale = amax/448.
* E4M3 causal prefill -- the causal prefill shapes with Q, K and V all given as
  E4M3 codes, each tensor with its own amax/448 scale (the same page, What:
  grouped E4M3 FP32 long-context operator).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HQ, HKV, D = 6, 1, 256
SCALE = 1.0 / 16.0


def _normal16(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------- causal prefill
@dataclass(frozen=True)
class CausalConfig:
    name: str
    nq: int
    n_kv: int
    hq: int = HQ
    hkv: int = HKV
    d: int = D
    scale: float = SCALE

    @property
    def q_pos0(self) -> int:
        return self.n_kv - self.nq


TINY = CausalConfig("tiny_q256_kv1024", nq=256, n_kv=1024)
LONG_40K = CausalConfig("long_q8000_kv40000", nq=8000, n_kv=40000)
SWEEP = tuple(CausalConfig(f"long_q8000_kv{kv}", nq=8000, n_kv=kv) for kv in range(48000, 128001, 8000))
HEADLINE = SWEEP[-1]  # Q=8000, KV=128000


def causal_inputs(nq: int, n_kv: int, seed: int, hq: int = HQ, hkv: int = HKV, d: int = D):
    """q [nq, hq, d], k [n_kv, hkv, d], v [n_kv, hkv, d] as fp16 numpy arrays."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (nq, hq, d))
    k = _normal16(rng, (n_kv, hkv, d))
    v = _normal16(rng, (n_kv, hkv, d))
    return q, k, v


# ------------------------------------------------------------- varlen prefill
@dataclass
class VarlenInputs:
    q: np.ndarray        # fp16 [total_q, hq, d]
    k: np.ndarray        # fp16 [total_kv, hkv, d]
    v: np.ndarray
    cu_q: np.ndarray     # int32 [batch + 1]
    cu_kv: np.ndarray    # int32 [batch + 1]
    scale: float = SCALE


def varlen_inputs(kv_lens, q_lens, seed: int, hq: int = HQ, hkv: int = HKV, d: int = D) -> VarlenInputs:
    """A batch of sequences packed end to end: sequence i has kv_lens[i] keys and
    q_lens[i] <= kv_lens[i] queries (its last positions).  Q, K, V are drawn in
    that order from one seeded N(0,1) float32 stream and rounded to fp16."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if (q_lens > kv_lens).any() or (q_lens < 0).any():
        raise ValueError("each sequence needs 0 <= q_len <= kv_len")
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    q = _normal16(rng, (int(cu_q[-1]), hq, d))
    k = _normal16(rng, (int(cu_kv[-1]), hkv, d))
    v = _normal16(rng, (int(cu_kv[-1]), hkv, d))
    return VarlenInputs(q=q, k=k, v=v, cu_q=cu_q, cu_kv=cu_kv)


def varlen_batch_lengths(seed: int, batch: int = 8, kv_lo: int = 4096, kv_hi: int = 32768, q_frac: float = 0.25):
    """Seeded request mix of a chunked-prefill batch: kv lengths uniform in
    [kv_lo, kv_hi], each request prefilling the last q_frac of its tokens."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(kv_lo, kv_hi + 1, size=batch)
    q = np.maximum(1, (kv * q_frac).astype(np.int64))
    return kv, q


# ------------------------------------------------------- paged block-sparse prefill
PAGE_SIZE = 16
KV_BLOCK_TOKENS = 4
QBLOCK_ROWS = 64
PAGE_POOL = 512


@dataclass
class PagedSparseInputs:
    q: np.ndarray            # fp16 [nq, hq, d]
    k_cache: np.ndarray      # fp16 [n_pages, page_size, hkv, d]
    v_cache: np.ndarray
    page_table: np.ndarray   # int32 [n_table]
    qblock_offsets: np.ndarray  # int32 [n_qblocks + 1]
    kv_block_ids: np.ndarray    # int32 [offsets[-1]]
    q_pos0: int
    live_len: int
    page_size: int = PAGE_SIZE
    kv_block_tokens: int = KV_BLOCK_TOKENS
    qblock_rows: int = QBLOCK_ROWS
    scale: float = SCALE
    meta: dict = field(default_factory=dict)


def paged_sparse_inputs(select_tokens: int, tail: int, seed: int, nq: int = 4096, n_pages: int | None = None,
                        poison_stale: bool = False, saturate: bool = False, identity_table: bool = False,
                        page_size: int = PAGE_SIZE, hq: int = HQ, hkv: int = HKV, d: int = D) -> PagedSparseInputs:
    """Paged block-sparse prefill inputs.

    Query row r sits at position tail + r, so the request holds ``tail`` tokens
    of earlier context and live_len = tail + nq.  The page table maps the
    ceil(live_len / page_size) logical pages to distinct physical pages drawn
    as a seeded random permutation of the pool (non-monotonic); the pool holds
    512 pages at page size 16 and twice the pages the request needs otherwise.  Query block b (rows
    64b..64b+63) always selects the 4-token block holding the position of its
    last row (its causal-diagonal block, of which only part may be visible: the
    partial tail), plus min(select_tokens/4 - 1, diag) distinct random earlier
    blocks (all earlier blocks when ``saturate``), emitted in shuffled order.
    With ``poison_stale`` every cache slot that holds no live token is NaN.
    """
    if select_tokens % KV_BLOCK_TOKENS or select_tokens < KV_BLOCK_TOKENS:
        raise ValueError("selection must be a positive multiple of the block size")
    if page_size % KV_BLOCK_TOKENS or page_size <= 0:
        raise ValueError("page size must be a positive multiple of the block size")
    rng = np.random.default_rng(seed)
    live_len = tail + nq
    n_table = -(-live_len // page_size)
    if n_pages is None:
        n_pages = PAGE_POOL if page_size == PAGE_SIZE else 2 * n_table
    q = _normal16(rng, (nq, hq, d))
    k_cache = _normal16(rng, (n_pages, page_size, hkv, d))
    v_cache = _normal16(rng, (n_pages, page_size, hkv, d))
    if n_table > n_pages:
        raise ValueError("page pool too small")
    perm = rng.permutation(n_pages)
    page_table = (np.arange(n_table) if identity_table else perm[:n_table]).astype(np.int32)
    if poison_stale:
        live = np.zeros((n_pages, page_size), dtype=bool)
        toks = np.arange(live_len)
        live[page_table[toks // page_size], toks % page_size] = True
        k_cache[~live] = np.float16(np.nan)
        v_cache[~live] = np.float16(np.nan)
    n_qblocks = -(-nq // QBLOCK_ROWS)
    offsets = [0]
    ids = []
    for b in range(n_qblocks):
        last_pos = tail + min(nq, (b + 1) * QBLOCK_ROWS) - 1
        diag = last_pos // KV_BLOCK_TOKENS
        n_extra = diag if saturate else min(select_tokens // KV_BLOCK_TOKENS - 1, diag)
        extra = rng.choice(diag, size=n_extra, replace=False) if n_extra > 0 else np.zeros(0, dtype=np.int64)
        sel = np.concatenate([[diag], extra]).astype(np.int64)
        rng.shuffle(sel)
        ids.append(sel)
        offsets.append(offsets[-1] + sel.size)
    return PagedSparseInputs(
        q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
        qblock_offsets=np.asarray(offsets, dtype=np.int32),
        kv_block_ids=np.concatenate(ids).astype(np.int32),
        q_pos0=tail, live_len=live_len, page_size=page_size,
        meta=dict(select_tokens=select_tokens, tail=tail, seed=seed, nq=nq, n_pages=n_pages,
                  poison_stale=poison_stale, saturate=saturate, page_size=page_size),
    )


def paged_large_table_inputs(n_table: int, n_pages: int, n_select: int, n_repeat: int, seed: int, nq: int = 128,
                             page_size: int = PAGE_SIZE, hq: int = HQ, hkv: int = HKV,
                             d: int = D) -> PagedSparseInputs:
    """Paged inputs for a long request held in a small pool: n_table logical pages of
    page_size tokens, each mapped to a physical page drawn at random from n_pages (pages are
    shared, so the cache stays small).  The nq query rows are the last nq positions; each
    query block selects its diagonal block plus n_select - 1 distinct random earlier blocks
    spread over the whole table, then n_repeat copies of already selected ids inserted at
    random places, in shuffled order."""
    rng = np.random.default_rng(seed)
    live_len = n_table * page_size
    q_pos0 = live_len - nq
    q = _normal16(rng, (nq, hq, d))
    k_cache = _normal16(rng, (n_pages, page_size, hkv, d))
    v_cache = _normal16(rng, (n_pages, page_size, hkv, d))
    page_table = rng.integers(0, n_pages, size=n_table).astype(np.int32)
    n_qblocks = -(-nq // QBLOCK_ROWS)
    offsets, ids = [0], []
    for b in range(n_qblocks):
        diag = (q_pos0 + min(nq, (b + 1) * QBLOCK_ROWS) - 1) // KV_BLOCK_TOKENS
        extra = rng.choice(diag, size=n_select - 1, replace=False)
        sel = list(np.concatenate([[diag], extra]))
        rng.shuffle(sel)
        for r in rng.choice(sel, size=n_repeat, replace=True) if n_repeat else []:
            sel.insert(int(rng.integers(0, len(sel) + 1)), r)
        ids.append(np.asarray(sel, dtype=np.int64))
        offsets.append(offsets[-1] + len(sel))
    return PagedSparseInputs(
        q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
        qblock_offsets=np.asarray(offsets, dtype=np.int32),
        kv_block_ids=np.concatenate(ids).astype(np.int32),
        q_pos0=q_pos0, live_len=live_len, page_size=page_size,
        meta=dict(n_table=n_table, n_pages=n_pages, n_select=n_select, n_repeat=n_repeat, seed=seed, nq=nq),
    )


# ------------------------------------------------------------ FP8 verifier tail
VERIFY_CONTEXT = 261888
E4M3_MAX = 448.0


@dataclass
class VerifyInputs:
    q: np.ndarray        # fp16 [nq, hq, d]
    k_bytes: np.ndarray  # uint8 [L, hkv, d]
    v_bytes: np.ndarray
    k_scale: float
    v_scale: float
    scale: float = SCALE


def _to_e4m3(x: np.ndarray, scale: np.float32) -> np.ndarray:
    import torch  # the float8 cast is a library primitive used only to make inputs

    y = np.clip(x / scale, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def verify_inputs(nq: int, context: int, seed: int, hq: int = HQ, hkv: int = HKV, d: int = D) -> VerifyInputs:
    """Verifier-tail inputs: fp16 Q and E4M3-coded K/V from N(0,1) draws."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (nq, hq, d))
    kf = rng.standard_normal((context, hkv, d), dtype=np.float32)
    vf = rng.standard_normal((context, hkv, d), dtype=np.float32)
    k_scale = np.float32(np.abs(kf).max() / np.float32(E4M3_MAX))
    v_scale = np.float32(np.abs(vf).max() / np.float32(E4M3_MAX))
    kb = _to_e4m3(kf, k_scale)
    del kf
    vb = _to_e4m3(vf, v_scale)
    return VerifyInputs(q=q, k_bytes=kb, v_bytes=vb, k_scale=float(k_scale), v_scale=float(v_scale))


# ------------------------------------------------------- E4M3 causal prefill
@dataclass
class E4M3PrefillInputs:
    q_bytes: np.ndarray  # uint8 [nq, hq, d] E4M3 codes
    k_bytes: np.ndarray  # uint8 [n_kv, hkv, d]
    v_bytes: np.ndarray
    q_scale: float
    k_scale: float
    v_scale: float
    q_pos0: int
    scale: float = SCALE


def e4m3_prefill_inputs(nq: int, n_kv: int, seed: int, hq: int = HQ, hkv: int = HKV, d: int = D) -> E4M3PrefillInputs:
    """Causal prefill inputs with Q, K and V all as E4M3 codes: N(0,1) float32
    draws in the order Q, K, V, each tensor quantised with its own scale
    amax/448 (the verifier-tail recipe applied to Q as well); the nq query rows
    sit at the last positions of the n_kv keys."""
    rng = np.random.default_rng(seed)
    out = []
    for shape in ((nq, hq, d), (n_kv, hkv, d), (n_kv, hkv, d)):
        x = rng.standard_normal(shape, dtype=np.float32)
        s = np.float32(np.abs(x).max() / np.float32(E4M3_MAX))
        out.append((_to_e4m3(x, s), float(s)))
        del x
    (qb, qs), (kb, ks), (vb, vs) = out
    return E4M3PrefillInputs(q_bytes=qb, k_bytes=kb, v_bytes=vb, q_scale=qs, k_scale=ks, v_scale=vs,
                             q_pos0=n_kv - nq)
