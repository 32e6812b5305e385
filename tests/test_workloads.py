"""Host-side checks of the seeded input generators (shapes, geometry, determinism)."""

import numpy as np

import workloads


def test_causal_inputs_shape_and_determinism():
    q, k, v = workloads.causal_inputs(8, 32, seed=0)
    assert q.shape == (8, 6, 256) and k.shape == (32, 1, 256) and v.shape == (32, 1, 256)
    assert q.dtype == np.float16
    q2, k2, v2 = workloads.causal_inputs(8, 32, seed=0)
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    assert workloads.HEADLINE.n_kv == 128000 and workloads.HEADLINE.q_pos0 == 120000
    assert [c.n_kv for c in workloads.SWEEP] == list(range(48000, 128001, 8000))


def test_paged_geometry():
    for tail in (0, 1, 2, 3):
        x = workloads.paged_sparse_inputs(select_tokens=64, tail=tail, seed=tail, nq=4096, d=8)
        assert x.live_len == 4096 + tail and x.q_pos0 == tail
        assert x.page_table.size == -(-x.live_len // 16)
        assert np.unique(x.page_table).size == x.page_table.size
        assert not np.all(np.diff(x.page_table) > 0)  # non-monotonic
        offs = x.qblock_offsets
        assert offs.size == 65 and offs[0] == 0
        for b in range(64):
            sel = x.kv_block_ids[offs[b]:offs[b + 1]]
            diag = (tail + 64 * b + 63) // 4
            assert sel.size == np.unique(sel).size
            assert diag in sel and sel.max() == diag
            assert sel.size == min(16, diag + 1)
        # diagonal block partial tail: the last row sees `tail` tokens of block 16b+16 (tail >= 1)
        if tail:
            assert (tail + 63) // 4 == 16
