"""GPU parity of gqa_prefill_paged_sparse against the fp64 oracle (through the C ABI)."""

import functools

import numpy as np
import pytest

import helpers
import oracle
import workloads
from helpers import to_dev, to_host

# The first rows of a query block can see as few as one selected token, so outputs
# with |O| >= 2 occur (one fp16 step there exceeds 1e-3);
# those elements are held to 1e-3 beyond their own fp16 rounding (helpers.assert_parity).
assert_parity = functools.partial(helpers.assert_parity, fp16_step_exempt=True)

pytestmark = pytest.mark.gpu


def _oracle(x, ids=None, offs=None, k_cache=None, v_cache=None, page_table=None):
    return oracle.prefill_paged_sparse(
        x.q, x.k_cache if k_cache is None else k_cache, x.v_cache if v_cache is None else v_cache,
        x.page_table if page_table is None else page_table, x.page_size,
        x.qblock_offsets if offs is None else offs, x.kv_block_ids if ids is None else ids, x.qblock_rows,
        x.kv_block_tokens, x.q_pos0, x.live_len, x.scale)[0]


def _gpu(x, ids=None, offs=None, k_cache=None, v_cache=None, page_table=None, want_ws=False):
    import gqa_causal_flash_amd as g

    out, ws = g.gqa_prefill_paged_sparse(
        to_dev(x.q), to_dev(x.k_cache if k_cache is None else k_cache),
        to_dev(x.v_cache if v_cache is None else v_cache), to_dev(x.page_table if page_table is None else page_table),
        to_dev(x.qblock_offsets if offs is None else offs), to_dev(x.kv_block_ids if ids is None else ids),
        x.q_pos0, x.live_len, x.scale)
    res = to_host(out)
    return (res, ws) if want_ws else res


@pytest.mark.parametrize("select", [64, 512, 2048])
@pytest.mark.parametrize("tail", [0, 1, 2, 3])
def test_paged_parity_config(select, tail):
    """4096 query rows, page-16 non-monotonic table, 4-token selection of S tokens, partial tail t."""
    x = workloads.paged_sparse_inputs(select_tokens=select, tail=tail, seed=100 * tail + select)
    assert_parity(_gpu(x), _oracle(x), f"S={select} t={tail}")


def test_paged_short_last_query_block_of_64():
    """4090 query tokens: 64 query blocks, the last one 58 tokens long, with selections long enough
    that query blocks are split between teams; the merge workgroups of the last query block have
    lanes past the last row."""
    x = workloads.paged_sparse_inputs(select_tokens=2048, tail=2, seed=8, nq=4090)
    assert x.qblock_offsets.size - 1 == 64
    assert_parity(_gpu(x), _oracle(x), "nq=4090")


def test_paged_128_entry_table():
    """The 128-entry page-16 table geometry: 2044 rows (short last query block)."""
    x = workloads.paged_sparse_inputs(select_tokens=512, tail=3, seed=7, nq=2044)
    assert x.page_table.size == 128
    assert_parity(_gpu(x), _oracle(x), "128-entry table")


def test_paged_hybrid_784_16_geometry():
    """Hybrid geometry: the cache is stored in pages of 784 tokens and addressed by a
    non-monotonic 128-entry page-16 table whose entries name 16-token sub-pages of
    those pages (784 = 49 x 16).  A 784-token page is 49 contiguous 16-token pages,
    so the page-16 path serves it over the same memory viewed as 49x as many pages."""
    n784 = 3
    x = workloads.paged_sparse_inputs(select_tokens=512, tail=3, seed=8, nq=2044, n_pages=49 * n784)
    assert x.page_table.size == 128 and x.page_table.max() < 49 * n784
    k784 = x.k_cache.reshape(n784, 784, 1, 256)  # the storage as 784-token pages
    v784 = x.v_cache.reshape(n784, 784, 1, 256)
    # the sub-page view addresses the same tokens as (page p // 49, offset 16 (p % 49) + j)
    pg = x.page_table
    toks = np.arange(x.live_len)
    sub = pg[toks // 16]
    assert np.array_equal(k784[sub // 49, 16 * (sub % 49) + toks % 16], x.k_cache[sub, toks % 16])
    out = _gpu(x, k_cache=k784.reshape(-1, 16, 1, 256), v_cache=v784.reshape(-1, 16, 1, 256))
    assert_parity(out, _oracle(x), "hybrid 784/16")


def test_paged_stale_poison():
    """NaN in every cache slot holding no live token changes nothing and stays out of the output."""
    x = workloads.paged_sparse_inputs(select_tokens=512, tail=2, seed=11)
    xp = workloads.paged_sparse_inputs(select_tokens=512, tail=2, seed=11, poison_stale=True)
    a, b = _gpu(x), _gpu(xp)
    assert np.isfinite(b).all()
    assert np.array_equal(a, b)
    assert_parity(b, _oracle(x), "poisoned")


def test_paged_identity_vs_permuted_table():
    """The same logical cache behind the identity page table and behind a permuted one."""
    x = workloads.paged_sparse_inputs(select_tokens=512, tail=1, seed=12)
    ref = _oracle(x)
    n_table = x.page_table.size
    toks = np.arange(n_table * 16)
    from oracle import attention as oatt

    k_log = oatt.gather_paged(x.k_cache, x.page_table, 16, toks).reshape(n_table, 16, 1, 256)
    v_log = oatt.gather_paged(x.v_cache, x.page_table, 16, toks).reshape(n_table, 16, 1, 256)
    ident = np.arange(n_table, dtype=np.int32)
    out_perm = _gpu(x)
    out_id = _gpu(x, k_cache=k_log, v_cache=v_log, page_table=ident)
    assert_parity(out_perm, ref, "permuted table")
    assert_parity(out_id, ref, "identity table")


def test_paged_saturated_matches_dense_causal():
    """Selecting every block up to the diagonal reproduces dense causal attention."""
    x = workloads.paged_sparse_inputs(select_tokens=64, tail=1, seed=13, nq=1024, saturate=True)
    out = _gpu(x)
    from oracle import attention as oatt

    toks = np.arange(x.live_len)
    kc = oatt.gather_paged(x.k_cache, x.page_table, 16, toks)
    vc = oatt.gather_paged(x.v_cache, x.page_table, 16, toks)
    ref, _ = oracle.prefill_causal(x.q, kc, vc, x.q_pos0, x.scale)
    assert_parity(out, ref, "saturated")


def test_paged_selection_longer_than_2048_blocks():
    """About 3000 blocks in one query block (128 rows at positions 12000.., every earlier block
    selected): the prepass's bitmap takes selections of any length."""
    x = workloads.paged_sparse_inputs(select_tokens=64, tail=12000, seed=41, nq=128, n_pages=1024, saturate=True)
    assert np.diff(x.qblock_offsets).min() > 2048
    assert_parity(_gpu(x), _oracle(x), "3000-block selections")


@pytest.mark.parametrize("select,tail", [(64, 0), (512, 1), (2048, 3)])
def test_paged_page784_parity(select, tail):
    """The block-sparse selection over a page-784 cache (non-monotonic table of 784-token pages)."""
    x = workloads.paged_sparse_inputs(select_tokens=select, tail=tail, seed=300 + select + tail, page_size=784)
    assert x.page_size == 784 and x.k_cache.shape[1] == 784
    assert_parity(_gpu(x), _oracle(x), f"page 784 S={select} t={tail}")


@pytest.mark.parametrize("page_size,select,tail", [(4, 512, 1), (12, 64, 3), (100, 2048, 2), (4096, 512, 0)])
def test_paged_page_size_extremes(page_size, select, tail):
    """Page sizes at both ends of the accepted range (one 4-token block per page, and 4096
    tokens per page) and two that are not powers of two, over 1000 query rows (short last
    query block)."""
    x = workloads.paged_sparse_inputs(select_tokens=select, tail=tail, seed=500 + page_size, nq=1000,
                                      page_size=page_size)
    assert x.k_cache.shape[1] == page_size
    assert_parity(_gpu(x), _oracle(x), f"page {page_size} S={select} t={tail}")


@pytest.mark.parametrize("page_size", [16, 784])
def test_paged_dense_causal_full_size(page_size):
    """Paged dense causal prefill (every block up to the diagonal selected), 4096 rows, against
    dense causal attention over the logical cache."""
    x = workloads.paged_sparse_inputs(select_tokens=64, tail=1, seed=31, saturate=True, page_size=page_size)
    out = _gpu(x)
    from oracle import attention as oatt

    toks = np.arange(x.live_len)
    kc = oatt.gather_paged(x.k_cache, x.page_table, page_size, toks)
    vc = oatt.gather_paged(x.v_cache, x.page_table, page_size, toks)
    ref, _ = oracle.prefill_causal(x.q, kc, vc, x.q_pos0, x.scale)
    assert_parity(out, ref, f"paged dense page {page_size}")


def test_paged_invalid_and_duplicate_entries_are_dropped():
    """Out-of-range block ids, out-of-range pages and duplicates contribute nothing and are counted."""
    import gqa_causal_flash_amd as g

    x = workloads.paged_sparse_inputs(select_tokens=64, tail=1, seed=14, nq=256)
    offs = x.qblock_offsets.astype(np.int64)
    ids = list(x.kv_block_ids)
    # block 0: add an id past the table; block 1: add a duplicate of its first id
    bad_id = x.page_table.size * 4 + 5
    new_ids = ids[:offs[1]] + [bad_id] + ids[offs[1]:offs[2]] + [ids[offs[1]]] + ids[offs[2]:]
    new_offs = offs.copy()
    new_offs[1:] += 1
    new_offs[2:] += 1
    new_ids = np.asarray(new_ids, dtype=np.int32)
    new_offs = new_offs.astype(np.int32)
    # a page-table entry out of range: make the table point one logical page at a missing physical page
    pt = x.page_table.copy()
    victim_page = 3 if ids[offs[1]] // 4 != 3 else 5
    pt[victim_page] = 10_000
    out, ws = _gpu(x, ids=new_ids, offs=new_offs, page_table=pt, want_ws=True)
    dropped = g.gqa_prefill_paged_sparse_dropped(ws)
    # reference: the same selection without the bad id and the duplicate, and without blocks of the victim page
    counts = []
    ref_ids = []
    for b in range(len(offs) - 1):
        sel = [i for i in x.kv_block_ids[offs[b]:offs[b + 1]] if i // 4 != victim_page]
        ref_ids += sel
        counts.append(len(sel))
    ref_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ref = _oracle(x, ids=np.asarray(ref_ids, dtype=np.int32), offs=ref_offs)
    n_victim = sum(1 for i in new_ids if i // 4 == victim_page)
    assert n_victim > 0
    assert dropped == 2 + n_victim
    assert_parity(out, ref, "dropped entries")


def test_paged_repeated_ids_are_dropped_across_the_whole_check_range():
    """Query blocks of 1800 distinct ids plus 200 repeats inserted at random places (drawn with
    replacement, so some ids occur three times): 2000 entries, so every one of the thread's four
    entry groups holds kept entries.  Each repeat is dropped and counted once, and the result equals
    the oracle on the selection as a set."""
    import gqa_causal_flash_amd as g

    x = workloads.paged_sparse_inputs(select_tokens=4 * 1800, tail=8000, seed=42, nq=128, n_pages=1024)
    rng = np.random.default_rng(43)
    offs = x.qblock_offsets
    ids, new_offs, n_rep = [], [0], 0
    for b in range(len(offs) - 1):
        sel = [int(i) for i in x.kv_block_ids[offs[b]:offs[b + 1]]]
        assert len(set(sel)) == len(sel) == 1800
        for r in rng.choice(sel, size=200, replace=True):
            sel.insert(int(rng.integers(0, len(sel) + 1)), int(r))
        n_rep += 200
        assert 1536 < len(sel) <= 2048
        ids += sel
        new_offs.append(len(ids))
    ids = np.asarray(ids, dtype=np.int32)
    new_offs = np.asarray(new_offs, dtype=np.int32)
    out, ws = _gpu(x, ids=ids, offs=new_offs, want_ws=True)
    assert g.gqa_prefill_paged_sparse_dropped(ws) == n_rep
    assert_parity(out, _oracle(x, ids=ids, offs=new_offs), "repeated ids")


@pytest.mark.parametrize("n_select,n_repeat", [(1500, 100), (3000, 0)])
def test_paged_table_beyond_the_bitmap(n_select, n_repeat):
    """A request of 70000 pages of 16 tokens (1.12M tokens, past the prepass bitmap's 262144
    blocks) held in a 64-page pool, selections spread over the whole table: 1500 ids plus 100
    repeats take the open-addressing path (each repeat dropped and counted), 3000 distinct ids the
    long path (given order)."""
    import gqa_causal_flash_amd as g

    x = workloads.paged_large_table_inputs(n_table=70000, n_pages=64, n_select=n_select, n_repeat=n_repeat,
                                           seed=50 + n_select)
    assert x.page_table.size * 4 > 262144
    out, ws = _gpu(x, want_ws=True)
    assert g.gqa_prefill_paged_sparse_dropped(ws) == n_repeat * 2
    assert_parity(out, _oracle(x), f"table beyond the bitmap S={n_select}")


def _subselect(x, counts, seed):
    """Per query block b, counts[b % len(counts)] distinct blocks drawn from the block's full causal
    selection (x built with saturate=True), in shuffled order."""
    rng = np.random.default_rng(seed)
    offs = x.qblock_offsets
    ids, new_offs = [], [0]
    for b in range(offs.size - 1):
        full = x.kv_block_ids[offs[b]:offs[b + 1]]
        k = min(counts[b % len(counts)], full.size)
        sel = rng.choice(full, size=k, replace=False) if k else np.zeros(0, dtype=np.int32)
        ids += [int(i) for i in sel]
        new_offs.append(len(ids))
    return np.asarray(ids, dtype=np.int32), np.asarray(new_offs, dtype=np.int32)


def test_paged_mixed_selection_lengths():
    """Selections of 0 to 1000 blocks mixed across 64 query blocks: empty query blocks between
    selected ones, single-block and part-filled sub-tiles, runs cut inside long blocks and boundaries
    moved to block ends."""
    x = workloads.paged_sparse_inputs(select_tokens=4, tail=2, seed=60, saturate=True)
    ids, offs = _subselect(x, [0, 1, 3, 8, 9, 16, 17, 64, 100, 511, 512, 513, 1000, 2, 0, 7], seed=61)
    assert (np.diff(offs) == 0).sum() >= 4
    assert_parity(_gpu(x, ids=ids, offs=offs), _oracle(x, ids=ids, offs=offs), "mixed selection lengths")


def test_paged_one_long_query_block_among_short_ones():
    """The last query block selects all of its 1024 blocks and every other one a single block, so the
    runs are at their shortest and the long block is split into about 26 pieces for the merge."""
    x = workloads.paged_sparse_inputs(select_tokens=4, tail=1, seed=62, saturate=True)
    ids, offs = _subselect(x, [1] * 63 + [4096], seed=63)
    assert np.diff(offs)[-1] == 1025
    assert_parity(_gpu(x, ids=ids, offs=offs), _oracle(x, ids=ids, offs=offs), "one long query block")


def test_paged_empty_selection_gives_zero_rows():
    x = workloads.paged_sparse_inputs(select_tokens=64, tail=0, seed=15, nq=128)
    offs = np.array([0, 0, x.qblock_offsets[2] - x.qblock_offsets[1]], dtype=np.int32)
    ids = x.kv_block_ids[x.qblock_offsets[1]:x.qblock_offsets[2]]
    out = _gpu(x, ids=ids, offs=offs)
    assert np.array_equal(out[:64], np.zeros_like(out[:64]))
    assert_parity(out, _oracle(x, ids=ids, offs=offs), "empty block 0")


def test_paged_deterministic():
    x = workloads.paged_sparse_inputs(select_tokens=2048, tail=3, seed=16)
    assert np.array_equal(_gpu(x), _gpu(x))


def test_paged_pool_at_the_32_bit_limit():
    """A page pool of 524287 pages of 16 tokens, the most whose K and V bytes fit 32-bit buffer offsets
    (2^32 - 8192 bytes each).  The request's pages are placed at the top of the pool through the page
    table, so every gathered row lies above 2^31 bytes; the result must equal the oracle on the same
    logical cache held in a small pool."""
    import torch

    import gqa_causal_flash_amd as g

    x = workloads.paged_sparse_inputs(select_tokens=512, tail=1, seed=31, nq=1024)
    n_big = 524287
    base = n_big - x.k_cache.shape[0]  # small page i lives at big page base + i
    k_big = torch.zeros((n_big,) + x.k_cache.shape[1:], dtype=torch.float16, device="cuda")
    v_big = torch.zeros_like(k_big)
    k_big[base:] = to_dev(x.k_cache)
    v_big[base:] = to_dev(x.v_cache)
    table = (x.page_table.astype(np.int64) + base).astype(np.int32)
    out, _ = g.gqa_prefill_paged_sparse(to_dev(x.q), k_big, v_big, to_dev(table), to_dev(x.qblock_offsets),
                                        to_dev(x.kv_block_ids), x.q_pos0, x.live_len, x.scale)
    res = to_host(out)
    del k_big, v_big
    assert_parity(res, _oracle(x), "pool of 524287 pages, request at the top")
