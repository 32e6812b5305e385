"""Calls on different streams run concurrently and independently.

The library keeps no mutable state between calls: each call works only in
the buffers and the workspace it is given, on the stream it is given.  Here
two dense prefills, a verifier call and a paged call, each with its own
output and workspace, are enqueued on two side streams at once (several
rounds, with the outputs poisoned with NaN in between), and every result is
compared bit for bit with the same call made alone on the current stream."""

import numpy as np
import pytest

import workloads
from helpers import to_dev

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_two_streams_match_serial_calls():
    import torch

    import gqa_causal_flash_amd as g

    # inputs: two dense prefills that are split into pieces (workspace + merge), one verifier, one paged call
    calls = []
    for nq, n_kv, seed in ((512, 9000, 31), (768, 20000, 32)):
        q, k, v = (to_dev(x) for x in workloads.causal_inputs(nq, n_kv, seed=seed))
        q_pos0 = n_kv - nq
        ws = torch.empty(max(1, g.gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0)), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty_like(q)
        calls.append((out, lambda o=None, w=None, q=q, k=k, v=v, q_pos0=q_pos0:
                      g.gqa_prefill_causal(q, k, v, q_pos0, workloads.SCALE, o=o, workspace=w), ws))

    xv = workloads.verify_inputs(4, 30000, seed=33)
    vq, kb, vb = to_dev(xv.q), to_dev(xv.k_bytes), to_dev(xv.v_bytes)
    vws = torch.empty(g.gqa_verify_fp8kv_workspace_size(4, 30000), dtype=torch.uint8, device="cuda")
    calls.append((torch.empty_like(vq), lambda o=None, w=None:
                  g.gqa_verify_fp8kv(vq, kb, vb, xv.k_scale, xv.v_scale, xv.scale, o=o, workspace=w), vws))

    xp = workloads.paged_sparse_inputs(select_tokens=512, tail=1, seed=34)
    dev = {n: to_dev(np.ascontiguousarray(getattr(xp, n)))
           for n in ("q", "k_cache", "v_cache", "page_table", "qblock_offsets", "kv_block_ids")}
    pws = torch.empty(g.gqa_prefill_paged_sparse_workspace_size(xp.q.shape[0], xp.kv_block_ids.size),
                      dtype=torch.uint8, device="cuda")
    calls.append((torch.empty_like(dev["q"]), lambda o=None, w=None:
                  g.gqa_prefill_paged_sparse(dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
                                             dev["qblock_offsets"], dev["kv_block_ids"], xp.q_pos0, xp.live_len,
                                             xp.scale, o=o, workspace=w)[0], pws))

    # each call alone on the current stream
    serial = []
    for _, fn, _ in calls:
        serial.append(fn().clone())
        torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for rnd in range(3):
        for out, _, _ in calls:
            out.fill_(float("nan"))
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for i, (out, fn, ws) in enumerate(calls):
            with torch.cuda.stream(streams[i % 2]):
                fn(out, ws)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i, ((out, _, _), ref) in enumerate(zip(calls, serial)):
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"round {rnd}, call {i}"
