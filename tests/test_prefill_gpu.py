"""GPU parity of gqa_prefill_causal against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_parity, to_dev, to_host

pytestmark = pytest.mark.gpu

SCALE = workloads.SCALE


def _gpu(q, k, v, q_pos0):
    import gqa_causal_flash_amd as g

    return to_host(g.gqa_prefill_causal(to_dev(q), to_dev(k), to_dev(v), q_pos0, SCALE))


@pytest.mark.parametrize(
    "nq,n_kv,q_pos0",
    [
        (256, 1024, 768),   # the tiny configuration
        (1, 1, 0),          # one query, one key
        (1, 200, 199),      # one query at the end
        (7, 100, 93),       # ragged: 42 packed rows, partial tiles
        (300, 300, 0),      # square causal from position 0
        (64, 1000, 500),    # queries in the middle (keys after them exist)
        (777, 2500, 1723),  # several q-blocks, ragged last block
        (256, 40000, 39744),  # few q-blocks over a long key range: many splits, merge path
        (1300, 4300, 3000),  # 128-row q-blocks at their largest (the 256-row schedule has 248 pieces)
        (2100, 4300, 2200),  # 256-row q-blocks (400 pieces), ragged last block, merge path
    ],
)
def test_prefill_parity(nq, n_kv, q_pos0):
    q, k, v = workloads.causal_inputs(nq, n_kv, seed=nq + n_kv)
    out = _gpu(q, k, v, q_pos0)
    ref, _ = oracle.prefill_causal(q, k, v, q_pos0, SCALE)
    assert_parity(out, ref, f"nq={nq} n_kv={n_kv} q_pos0={q_pos0}")


def test_prefill_ignores_keys_after_last_query():
    """K/V rows after the last query position never take part (NaN there changes nothing)."""
    nq, n_kv, q_pos0 = 100, 700, 300
    q, k, v = workloads.causal_inputs(nq, n_kv, seed=5)
    base = _gpu(q, k, v, q_pos0)
    k2, v2 = k.copy(), v.copy()
    k2[q_pos0 + nq:] = np.float16(np.nan)
    v2[q_pos0 + nq:] = np.float16(np.nan)
    out = _gpu(q, k2, v2, q_pos0)
    assert np.isfinite(out).all()
    assert np.array_equal(out, base)


def test_prefill_deterministic():
    nq, n_kv = 512, 9000
    q, k, v = workloads.causal_inputs(nq, n_kv, seed=9)
    a = _gpu(q, k, v, n_kv - nq)
    b = _gpu(q, k, v, n_kv - nq)
    assert np.array_equal(a, b)


# At these sizes the kernel works on q-blocks of 256 packed rows (token * 6 + head);
# a test that covers complete q-blocks covers every key-range piece and merge of each.
# (Workloads too small to give every compute unit a piece take 128-row q-blocks:
# the tiny configuration and most cases of test_prefill_parity.)
QBLOCK_PACKED_ROWS = 256
WHOLE_TENSOR_KV = (40000, 128000)  # the page's two printed points (Test Result)


def qblock_tokens(nq, blocks, hq=6):
    """Query tokens whose packed rows meet the given q-blocks (every row of each block)."""
    toks = set()
    for b in blocks:
        r0, r1 = QBLOCK_PACKED_ROWS * b, min(hq * nq, QBLOCK_PACKED_ROWS * (b + 1))
        toks.update(range(r0 // hq, (r1 - 1) // hq + 1))
    return np.array(sorted(toks), dtype=np.int64)


@pytest.mark.parametrize("cfg", (workloads.LONG_40K,) + workloads.SWEEP, ids=lambda c: c.name)
def test_prefill_full_size(cfg):
    """Full-size long prefill at every point of the key sweep (KV = 40000, 48000..128000, Q = 8000 at the
    last positions) in the benchmark's launch configuration.  At KV = 40000 and 128000 the whole output is
    compared; at the other points, every row of the first, the last and every 16th q-block."""
    from oracle import rowpool

    q, k, v = workloads.causal_inputs(cfg.nq, cfg.n_kv, seed=0)
    print(f"[full size] {cfg.name}: GPU", flush=True)
    out = _gpu(q, k, v, cfg.q_pos0)
    assert np.isfinite(out).all()
    if cfg.n_kv in WHOLE_TENSOR_KV:
        rows = np.arange(cfg.nq)
    else:
        nqb = -(-6 * cfg.nq // QBLOCK_PACKED_ROWS)
        rows = qblock_tokens(cfg.nq, sorted(set(range(0, nqb, 16)) | {nqb - 1}))
    print(f"[full size] {cfg.name}: oracle on {rows.size} rows, {rowpool.host_cores()} processes", flush=True)
    ref, _ = rowpool.run_rows("prefill_causal", (q, k, v, cfg.q_pos0, SCALE), rows=rows)
    assert_parity(out[rows], ref, f"{cfg.name} ({rows.size} of {cfg.nq} rows)")


def test_prefill_profiling_times_and_clock():
    """Profiling brackets the main kernel and samples the shader clock; results are unchanged."""
    import gqa_causal_flash_amd as g

    nq, n_kv = 512, 9000
    q, k, v = workloads.causal_inputs(nq, n_kv, seed=9)
    plain = _gpu(q, k, v, n_kv - nq)
    g.gqa_profile_start()
    profiled = _gpu(q, k, v, n_kv - nq)
    ms, n = g.gqa_profile_stop()
    mhz = g.gqa_profile_clock_mhz()
    assert np.array_equal(plain, profiled)
    assert n == 1 and ms > 0
    assert 300.0 < mhz < 3000.0, mhz


def test_prefill_at_the_32_bit_key_limit():
    """8388607 keys, the most whose K and V bytes fit 32-bit buffer offsets (2^32 - 512 bytes each),
    with six query rows at the last positions.  K is zero except for its last 4096 keys, so each
    row's keys split exactly into a prefix of equal scores (mean of V, log-sum-exp log(count): the
    zero-K closed form) and a tail that the oracle evaluates; the two are merged by log-sum-exp.
    V is random everywhere, so every key's row must be read from the right place."""
    n_kv, nq, tail = 8388607, 6, 4096
    q_pos0 = n_kv - nq
    prefix = n_kv - tail
    rng = np.random.default_rng(77)
    q = workloads._normal16(rng, (nq, 6, 256))
    k = np.zeros((n_kv, 1, 256), dtype=np.float16)
    k[prefix:] = workloads._normal16(rng, (tail, 1, 256))
    v = np.empty((n_kv, 1, 256), dtype=np.float16)
    vsum = np.zeros(256, dtype=np.float64)
    step = 1 << 19
    for a in range(0, n_kv, step):
        b = min(n_kv, a + step)
        v[a:b] = workloads._normal16(rng, (b - a, 1, 256))
        vsum += v[a:min(b, prefix), 0].astype(np.float64).sum(axis=0) if a < prefix else 0.0
    print("[32-bit limit] inputs ready", flush=True)
    out = _gpu(q, k, v, q_pos0)
    print("[32-bit limit] GPU done", flush=True)

    qf = q.reshape(nq * 6, 256)
    pos = q_pos0 + np.repeat(np.arange(nq), 6)
    vis = oracle.causal_visible(pos, np.arange(prefix, n_kv))
    o_t, lse_t = oracle.attend(qf, k[prefix:, 0], v[prefix:, 0], vis, SCALE)
    lse_p = np.log(prefix)
    mx = np.maximum(lse_t, lse_p)
    w_p, w_t = np.exp(lse_p - mx), np.exp(lse_t - mx)
    ref = (w_p[:, None] * (vsum / prefix)[None, :] + w_t[:, None] * o_t) / (w_p + w_t)[:, None]
    assert_parity(out.reshape(nq * 6, 256), ref, "n_kv=8388607 q=6")
