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


@pytest.mark.parametrize("nq", [2, 4, 8])
def test_verify_parity_full_context(nq):
    """Verifier tail of 2/4/8 rows at context 261888 (E4M3 K/V, per-tensor scales)."""
    x = workloads.verify_inputs(nq, workloads.VERIFY_CONTEXT, seed=nq)
    assert_parity(_gpu(x), _oracle(x), f"q={nq} ctx=261888")


@pytest.mark.parametrize("nq,ctx", [(1, 1), (1, 33), (5, 100), (8, 8), (8, 1000), (3, 4097), (6, 262144)])
def test_verify_parity_edges(nq, ctx):
    x = workloads.verify_inputs(nq, ctx, seed=nq * 7 + ctx)
    assert_parity(_gpu(x), _oracle(x), f"q={nq} ctx={ctx}")


def test_verify_deterministic():
    x = workloads.verify_inputs(8, 50000, seed=3)
    assert np.array_equal(_gpu(x), _gpu(x))
