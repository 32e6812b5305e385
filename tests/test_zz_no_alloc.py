"""gqa_verify_fp8kv_noalloc: the verifier tail with its partials in the library's fixed per-device
scratch instead of a caller workspace, checked through the C ABI against gqa_verify_fp8kv."""

import numpy as np
import pytest

import workloads
from helpers import to_host

pytestmark = pytest.mark.gpu


def _inputs(nq, ctx, seed):
    import torch

    x = workloads.verify_inputs(nq, ctx, seed)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return x, dev(x.q), dev(x.k_bytes), dev(x.v_bytes)


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    """Two calls in a row on the shared scratch, the second with a smaller input (fewer rows, a much shorter
    context, so fewer partial slots), each equal bit for bit to the entry point with its own workspace
    (same kernels, same schedule).  Neither call allocates through torch's allocator."""
    import torch

    import gqa_causal_flash_amd as g

    cases = [(8, workloads.VERIFY_CONTEXT, 0), (2, 5000, 1)]
    prepared = [_inputs(*c) for c in cases]
    outs = [torch.empty_like(q) for _, q, _, _ in prepared]
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for (x, q, k, v), o in zip(prepared, outs):
        print(f"[no-alloc] nq={q.shape[0]} ctx={k.shape[0]}", flush=True)
        g.gqa_verify_fp8kv_noalloc(q, k, v, x.k_scale, x.v_scale, x.scale, o=o)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for (x, q, k, v), o in zip(prepared, outs):
        ref = to_host(g.gqa_verify_fp8kv(q, k, v, x.k_scale, x.v_scale, x.scale))
        got = to_host(o)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref), f"nq={q.shape[0]} ctx={k.shape[0]}"


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    """Contexts beyond the verifier's 262144-token capability are refused before anything runs."""
    import torch

    import gqa_causal_flash_amd as g

    q = torch.zeros((2, 6, 256), dtype=torch.float16, device="cuda")
    k = torch.zeros((262145, 1, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(g.GQAError) as e:
        g.gqa_verify_fp8kv_noalloc(q, k, k, 1.0, 1.0, 0.0625)
    assert e.value.status == g.GQA_ERR_UNSUPPORTED
