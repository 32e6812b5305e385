"""GPU parity of gqa_prefill_causal_varlen (packed batch, per-row lse) against the fp64 oracle."""

import functools

import numpy as np
import pytest

import helpers
import oracle
import workloads
from helpers import to_dev, to_host

# The first rows of a sequence that starts at position 0 see one to a few keys, so
# outputs with |O| >= 2 occur (one fp16 step there exceeds 1e-3);
# those elements are held to 1e-3 beyond their own fp16 rounding (helpers.assert_parity).
assert_parity = functools.partial(helpers.assert_parity, fp16_step_exempt=True)

pytestmark = pytest.mark.gpu

# lse: the fp16 weights the kernel sums differ from the exact ones by <= 2^-11
# relative, so log l moves by <= 4.9e-4; 1e-3 leaves room for fp32 sums
TOL_LSE = 1e-3


def _gpu(x, cu_q=None, want_ws=False):
    import gqa_causal_flash_amd as g

    o, lse, ws = g.gqa_prefill_causal_varlen(to_dev(x.q), to_dev(x.k), to_dev(x.v),
                                             to_dev(x.cu_q if cu_q is None else cu_q), to_dev(x.cu_kv), x.scale)
    res = (to_host(o), lse.cpu().numpy())
    return res + (ws,) if want_ws else res


def _check(x, label):
    o, lse = _gpu(x)
    ref, ref_lse = oracle.prefill_causal_varlen(x.q, x.k, x.v, x.cu_q, x.cu_kv, x.scale)
    assert_parity(o, ref, label)
    assert np.isfinite(lse).all(), label
    err = np.abs(lse.astype(np.float64) - ref_lse).max()
    assert err <= TOL_LSE, f"{label}: lse error {err:.3e}"


@pytest.mark.parametrize("kv,q", [
    ([300, 1, 0, 1000, 257], [300, 1, 0, 77, 5]),   # nq = nkv, one key, empty, partial q-blocks
    ([5000, 4096, 33], [4096, 1, 33], ),            # one-row sequence next to long ones
    ([20000, 9000, 33000], [2000, 9000, 4000]),     # split over keys, merged
])
def test_varlen_parity(kv, q):
    x = workloads.varlen_inputs(kv, q, seed=sum(kv) + len(q))
    _check(x, f"kv={kv} q={q}")


def test_varlen_many_sequences():
    rng = np.random.default_rng(5)
    kv = rng.integers(1, 3000, size=37)
    q = np.array([rng.integers(0, k + 1) for k in kv])
    _check(workloads.varlen_inputs(kv, q, seed=6), "37 sequences")


def test_varlen_unsplit_path_writes_lse():
    """Enough q-blocks that no sequence is split: the main kernel writes O and lse itself."""
    kv = [2000] * 30
    q = [1500] * 30  # 30 x ceil(9000 / 256) = 1080 q-blocks: four workgroups per CU without a split
    _check(workloads.varlen_inputs(kv, q, seed=8), "unsplit")


def test_varlen_single_sequence_matches_dense_oracle():
    x = workloads.varlen_inputs([9000], [512], seed=9)
    o, lse = _gpu(x)
    ref, ref_lse = oracle.prefill_causal(x.q, x.k, x.v, 9000 - 512, x.scale)
    assert_parity(o, ref, "B=1")
    assert np.abs(lse - ref_lse).max() <= TOL_LSE


def test_varlen_invalid_sequence_is_skipped_and_counted():
    """A sequence with more queries than keys is skipped and counted; the others are computed."""
    import gqa_causal_flash_amd as g

    kv, q = [400, 300, 500], [100, 50, 200]
    x = workloads.varlen_inputs(kv, q, seed=10)
    cu_kv = np.array([0, 400, 420, 920], dtype=np.int32)  # sequence 1: 50 queries, 20 keys
    o, lse, ws = g.gqa_prefill_causal_varlen(to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.cu_q), to_dev(cu_kv),
                                             x.scale)
    assert g.gqa_prefill_causal_varlen_skipped(ws) == 1
    o = to_host(o)
    ref0, _ = oracle.prefill_causal(x.q[0:100], x.k[0:400], x.v[0:400], 300, x.scale)
    ref2, _ = oracle.prefill_causal(x.q[150:350], x.k[420:920], x.v[420:920], 300, x.scale)
    assert_parity(o[0:100], ref0, "sequence 0")
    assert_parity(o[150:350], ref2, "sequence 2")


def test_varlen_deterministic():
    x = workloads.varlen_inputs([7000, 3000], [1000, 3000], seed=12)
    a, la = _gpu(x)
    b, lb = _gpu(x)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_varlen_benchmark_batch_sampled_rows():
    """The benchmark's chunked-prefill batch (8 requests, seed 0) in the launch it times,
    checked on 16 sampled query tokens of every request against the causal oracle of
    that request's own slices (the definition the varlen pins fix)."""
    kv, ql = workloads.varlen_batch_lengths(0)
    x = workloads.varlen_inputs(kv, ql, 0)
    o, lse = _gpu(x)
    rng = np.random.default_rng(77)
    for i, (nkv, nq) in enumerate(zip(kv, ql)):
        q0, k0 = int(x.cu_q[i]), int(x.cu_kv[i])
        rows = np.unique(np.concatenate([[0, nq - 1], rng.choice(nq, 14, replace=False)]))
        ref, ref_lse = oracle.prefill_causal(x.q[q0:q0 + nq], x.k[k0:k0 + nkv], x.v[k0:k0 + nkv], int(nkv - nq),
                                             x.scale, rows=rows)
        assert_parity(o[q0 + rows], ref, f"request {i} (kv {nkv}, q {nq})")
        assert np.abs(lse[q0 + rows].astype(np.float64) - ref_lse).max() <= TOL_LSE, f"request {i} lse"


def test_varlen_sequence_at_the_32_bit_key_limit():
    """A packed key buffer of 8388607 rows, the most whose K and V bytes fit 32-bit buffer offsets: the
    first sequence holds keys only (no queries), the second its 1024 keys at the very top of the buffer
    with 256 queries.  The result must equal the dense oracle of the second sequence alone."""
    import torch

    import gqa_causal_flash_amd as g

    total_kv, nkv, nq = 8388607, 1024, 256
    q, k, v = workloads.causal_inputs(nq, nkv, seed=41)
    k_big = torch.zeros((total_kv, 1, 256), dtype=torch.float16, device="cuda")
    v_big = torch.zeros_like(k_big)
    k_big[total_kv - nkv:] = to_dev(k)
    v_big[total_kv - nkv:] = to_dev(v)
    cu_q = np.array([0, 0, nq], dtype=np.int32)
    cu_kv = np.array([0, total_kv - nkv, total_kv], dtype=np.int32)
    o, lse, _ = g.gqa_prefill_causal_varlen(to_dev(q), k_big, v_big, to_dev(cu_q), to_dev(cu_kv), workloads.SCALE)
    res, res_lse = to_host(o), lse.cpu().numpy()
    del k_big, v_big
    ref, ref_lse = oracle.prefill_causal(q, k, v, nkv - nq, workloads.SCALE)
    assert_parity(res, ref, "varlen sequence at the top of 8388607 keys")
    err = np.abs(res_lse.astype(np.float64) - ref_lse).max()
    assert err <= TOL_LSE, f"lse error {err:.3e}"
