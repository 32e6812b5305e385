"""HIP graph capture of every entry point: replays are bitwise equal to eager calls.

Each call is captured once (through torch's graph capture of the current
stream) with device-resident inputs, outputs and workspace.  The graph is then
replayed several times with eager work between the replays (the output is
overwritten with NaN first, and the inputs are changed once), and every replay
is compared bit for bit with an eager call on the same inputs."""

import numpy as np
import pytest

import workloads
from helpers import to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the graph
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_matches(g, out, eager, refresh=None, replays=3):
    import torch

    for i in range(replays):
        if refresh is not None and i == replays - 1:
            eager = refresh()  # new input contents; the graph must read them
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


def test_graph_prefill_causal():
    import torch

    import gqa_causal_flash_amd as g

    nq, n_kv = 512, 9000  # split into pieces: main kernel + merge in the graph
    q, k, v = (to_dev(x) for x in workloads.causal_inputs(nq, n_kv, seed=21))
    q_pos0 = n_kv - nq
    ws = torch.empty(max(1, g.gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    eager = g.gqa_prefill_causal(q, k, v, q_pos0, workloads.SCALE).clone()
    graph = _capture(lambda: g.gqa_prefill_causal(q, k, v, q_pos0, workloads.SCALE, o=out, workspace=ws))

    def refresh():
        q.mul_(-0.5)
        return g.gqa_prefill_causal(q, k, v, q_pos0, workloads.SCALE).clone()

    _replay_matches(graph, out, eager, refresh)


def test_graph_paged_sparse():
    import torch

    import gqa_causal_flash_amd as g

    x = workloads.paged_sparse_inputs(select_tokens=512, tail=1, seed=22)
    dev = {n: to_dev(np.ascontiguousarray(getattr(x, n)))
           for n in ("q", "k_cache", "v_cache", "page_table", "qblock_offsets", "kv_block_ids")}
    ws = torch.empty(g.gqa_prefill_paged_sparse_workspace_size(x.q.shape[0], x.kv_block_ids.size),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])

    def call(o=None, w=None):
        return g.gqa_prefill_paged_sparse(dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
                                          dev["qblock_offsets"], dev["kv_block_ids"], x.q_pos0, x.live_len, x.scale,
                                          o=o, workspace=w)[0]

    eager = call().clone()
    graph = _capture(lambda: call(out, ws))

    def refresh():
        dev["q"].mul_(-0.5)
        return call().clone()

    _replay_matches(graph, out, eager, refresh)


@pytest.mark.parametrize("nq", [2, 8])
def test_graph_verify_fp8kv(nq):
    import torch

    import gqa_causal_flash_amd as g

    x = workloads.verify_inputs(nq, 20000, seed=23 + nq)
    q, kb, vb = to_dev(x.q), to_dev(x.k_bytes), to_dev(x.v_bytes)
    ws = torch.empty(g.gqa_verify_fp8kv_workspace_size(nq, 20000), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    eager = g.gqa_verify_fp8kv(q, kb, vb, x.k_scale, x.v_scale, x.scale).clone()
    graph = _capture(lambda: g.gqa_verify_fp8kv(q, kb, vb, x.k_scale, x.v_scale, x.scale, o=out, workspace=ws))

    def refresh():
        q.mul_(-0.5)
        return g.gqa_verify_fp8kv(q, kb, vb, x.k_scale, x.v_scale, x.scale).clone()

    _replay_matches(graph, out, eager, refresh)


def test_graph_prefill_causal_varlen():
    import torch

    import gqa_causal_flash_amd as g

    x = workloads.varlen_inputs([3000, 1, 5000], [700, 1, 2000], seed=24)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    cu_q, cu_kv = to_dev(x.cu_q), to_dev(x.cu_kv)
    ws = torch.empty(g.gqa_prefill_causal_varlen_workspace_size(3, q.shape[0]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], 6), dtype=torch.float32, device="cuda")
    eager = g.gqa_prefill_causal_varlen(q, k, v, cu_q, cu_kv, x.scale)[0].clone()
    graph = _capture(lambda: g.gqa_prefill_causal_varlen(q, k, v, cu_q, cu_kv, x.scale, o=out, lse=lse, workspace=ws))

    def refresh():
        q.mul_(-0.5)
        return g.gqa_prefill_causal_varlen(q, k, v, cu_q, cu_kv, x.scale)[0].clone()

    _replay_matches(graph, out, eager, refresh)


def test_graph_prefill_causal_e4m3():
    import torch

    import gqa_causal_flash_amd as g

    nq, n_kv = 512, 9000
    x = workloads.e4m3_prefill_inputs(nq, n_kv, seed=22)
    q8, k8, v8 = (torch.from_numpy(a).cuda() for a in (x.q_bytes, x.k_bytes, x.v_bytes))
    ws = torch.empty(max(1, g.gqa_prefill_causal_workspace_size(nq, n_kv, x.q_pos0)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((nq, 6, 256), dtype=torch.float16, device="cuda")
    call = lambda **kw: g.gqa_prefill_causal_e4m3(q8, x.q_scale, k8, x.k_scale, v8, x.v_scale, x.q_pos0, x.scale,
                                                  **kw)
    eager = call().clone()
    graph = _capture(lambda: call(o=out, workspace=ws))

    def refresh():
        k8.copy_(torch.from_numpy(workloads.e4m3_prefill_inputs(nq, n_kv, seed=23).k_bytes))
        return call()

    _replay_matches(graph, out, eager, refresh)
