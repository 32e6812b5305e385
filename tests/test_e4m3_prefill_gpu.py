"""GPU parity of gqa_prefill_causal_e4m3 (Q K^T on the FP8 matrix cores) against the
fp64 oracle of the quantised-Q definition, through the C ABI."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_parity, to_host

pytestmark = pytest.mark.gpu

E4M3_NAN = 0x7F  # S.1111.111


def _gpu(x, q_pos0=None, q_scale=None, v_scale=None, scale=None, k_bytes=None, v_bytes=None):
    import torch

    import gqa_causal_flash_amd as g

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = g.gqa_prefill_causal_e4m3(dev(x.q_bytes), x.q_scale if q_scale is None else q_scale,
                                  dev(x.k_bytes if k_bytes is None else k_bytes), x.k_scale,
                                  dev(x.v_bytes if v_bytes is None else v_bytes),
                                  x.v_scale if v_scale is None else v_scale,
                                  x.q_pos0 if q_pos0 is None else q_pos0, x.scale if scale is None else scale)
    return to_host(o)


def _ref(x, rows=None):
    o, _ = oracle.prefill_causal_e4m3(x.q_bytes, x.q_scale, x.k_bytes, x.k_scale, x.v_bytes, x.v_scale, x.q_pos0,
                                      x.scale, rows=rows)
    return o


@pytest.mark.parametrize(
    "nq,n_kv",
    [
        (256, 1024),    # the tiny configuration's shape
        (1, 1),         # one query, one key
        (7, 100),       # ragged: 42 packed rows, partial tiles
        (300, 300),     # square causal from position 0
        (777, 2500),    # several q-blocks, ragged last block
        (256, 40000),   # few q-blocks over a long key range: key split and merge
    ],
)
def test_e4m3_prefill_parity(nq, n_kv):
    x = workloads.e4m3_prefill_inputs(nq, n_kv, seed=nq + 3 * n_kv)
    assert_parity(_gpu(x), _ref(x), f"e4m3 nq={nq} n_kv={n_kv}")


def test_e4m3_prefill_queries_in_the_middle():
    """Queries before the end of the key range: keys after the last query never take part."""
    x = workloads.e4m3_prefill_inputs(64, 1000, seed=61)
    x.q_pos0 = 500
    base = _gpu(x)
    assert_parity(base, _ref(x), "e4m3 q_pos0=500")
    k2, v2 = x.k_bytes.copy(), x.v_bytes.copy()
    k2[564:] = E4M3_NAN
    v2[564:] = E4M3_NAN
    out = _gpu(x, k_bytes=k2, v_bytes=v2)
    assert np.isfinite(out).all()
    assert np.array_equal(out, base)


def test_e4m3_prefill_scales_are_applied_exactly():
    """Powers of two moved between the Q scale and the softmax scale change nothing;
    doubling the V scale doubles O exactly."""
    x = workloads.e4m3_prefill_inputs(200, 3000, seed=62)
    base = _gpu(x)
    assert np.array_equal(_gpu(x, q_scale=2 * x.q_scale, scale=x.scale / 2), base)
    doubled = _gpu(x, v_scale=2 * x.v_scale).astype(np.float32)
    # exact wherever O is a normal fp16 number; subnormal outputs round on a grid
    # that does not scale with O, so there they agree to one subnormal step
    normal = np.abs(base.astype(np.float32)) >= 2.0 ** -14
    assert np.array_equal(doubled[normal], 2 * base.astype(np.float32)[normal])
    assert np.abs(doubled - 2 * base.astype(np.float32)).max() <= 2.0 ** -23


def test_e4m3_prefill_deterministic():
    x = workloads.e4m3_prefill_inputs(512, 9000, seed=63)
    assert np.array_equal(_gpu(x), _gpu(x))


@pytest.mark.parametrize("nq,n_kv", [(8000, 40000), (8000, 128000)])
def test_e4m3_prefill_full_size(nq, n_kv):
    """Full-size E4M3 long prefill in the benchmark's launch configuration, whole output."""
    from oracle import rowpool

    x = workloads.e4m3_prefill_inputs(nq, n_kv, seed=0)
    print(f"[full size] e4m3 q{nq} kv{n_kv}: GPU", flush=True)
    out = _gpu(x)
    assert np.isfinite(out).all()
    print(f"[full size] e4m3 q{nq} kv{n_kv}: oracle, {rowpool.host_cores()} processes", flush=True)
    ref, _ = rowpool.run_rows("prefill_causal_e4m3", (x.q_bytes, x.q_scale, x.k_bytes, x.k_scale, x.v_bytes,
                                                      x.v_scale, x.q_pos0, x.scale), n_rows=nq)
    assert_parity(out, ref, f"e4m3 q{nq} kv{n_kv} (whole output)")
