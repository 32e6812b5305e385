"""GPU parity of gqa_verify_fp8kv against the fp64 oracle fed the same E4M3 bytes."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_parity, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gpu(x):
    import gqa_causal_flash_amd as g

    out = g.gqa_verify_fp8kv(to_dev(x.q), to_dev(x.k_bytes), to_dev(x.v_bytes), x.k_scale, x.v_scale, x.scale)
    return to_host(out)


def _oracle(x):
    return oracle.verify_fp8kv(x.q, x.k_bytes, x.v_bytes, x.k_scale, x.v_scale, x.scale)[0]


@pytest.mark.parametrize("nq", [1, 2, 4, 8])
def test_verify_parity_full_context(nq):
    """Verifier tail of 1 (the single-row tail) and 2/4/8 rows at context 261888 (E4M3 K/V,
    per-tensor scales)."""
    x = workloads.verify_inputs(nq, workloads.VERIFY_CONTEXT, seed=nq)
    assert_parity(_gpu(x), _oracle(x), f"q={nq} ctx=261888")


@pytest.mark.parametrize("nq,ctx", [(1, 1), (1, 33), (5, 100), (6, 100), (8, 8), (8, 1000), (3, 4097), (7, 4097),
                                    (6, 262144)])
def test_verify_parity_edges(nq, ctx):
    """One 32-row block (q <= 5) and two (q = 6..8), with 1 to 16 tiles per workgroup, odd counts included."""
    x = workloads.verify_inputs(nq, ctx, seed=nq * 7 + ctx)
    assert_parity(_gpu(x), _oracle(x), f"q={nq} ctx={ctx}")


def test_verify_deterministic():
    x = workloads.verify_inputs(8, 50000, seed=3)
    assert np.array_equal(_gpu(x), _gpu(x))


def test_verify_decodes_every_e4m3_code_exactly():
    """One query row, one key: O equals the decoded V row, so all 256 codes (one per
    head-dim column) must come back as their exact values, NaN for 0x7F and 0xFF."""
    import gqa_causal_flash_amd as g

    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 6, 256)).astype(np.float16)
    kb = np.zeros((1, 1, 256), dtype=np.uint8)  # code 0 = +0: a finite score
    vb = np.arange(256, dtype=np.uint8).reshape(1, 1, 256)
    out = to_host(g.gqa_verify_fp8kv(to_dev(q), to_dev(kb), to_dev(vb), 1.0, 1.0, workloads.SCALE))
    want = oracle.e4m3_decode(vb[0, 0]).astype(np.float16)  # every E4M3 value is exact in fp16
    for h in range(6):
        got = out[0, h]
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), h
        # exact values (code 0x80, -0, comes back as +0: the accumulator starts at +0)
        assert np.array_equal(got[~nan], want[~nan]), h
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
