"""The entry points inside a captured HIP graph: the library enqueues kernel
launches only (no allocation, no memset, no synchronization), so a graph
captured from one call replays it.  Each replay follows eager work that
rewrites the inputs in place, and its output must equal an eager call's on
the same inputs, bit for bit."""
import numpy as np
import pytest
import torch

import precision_attention_qsdpa_amd as qs
from gpu_helpers import from_dev, to_dev
from workloads import WORKLOADS, draw

pytestmark = pytest.mark.gpu

N, H = 1000, 3


def _inputs(seed):
    return draw(WORKLOADS["tiny"], heads=H, seq_len=N, seed=seed)


def _replays_match_eager(call, params, fmt_label, out_of):
    """Capture ``call(q, k, v, out, ws, stream)`` once, then three times:
    copy new inputs into the captured buffers, replay, and compare with an
    eager call on fresh buffers."""
    q, k, v = (to_dev(x) for x in _inputs(700))
    out = torch.empty_like(q)
    ws = qs.empty_workspace(params)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, k, v, out, ws, side)   # first call: loads the library, looks up device symbols
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(q, k, v, out, ws, side)
    torch.cuda.synchronize()
    for seed in (701, 702, 703):
        qb, kb, vb = _inputs(seed)
        for dst, src in ((q, qb), (k, kb), (v, vb)):
            dst.copy_(to_dev(src))
        out.fill_(0)
        torch.cuda.synchronize()
        print(f"[graph] {fmt_label} replay with inputs seed {seed}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = from_dev(out)
        q2, k2, v2 = (to_dev(x) for x in (qb, kb, vb))
        want = out_of(q2, k2, v2)
        torch.cuda.synchronize()
        assert np.array_equal(got, want), f"{fmt_label}: replay with seed {seed} differs from the eager call"


@pytest.mark.parametrize("fmt", ["fp8", "fp4", "mxfp4"])
def test_forward_graph_replays_match_eager(gpu_lib, fmt):
    params = qs.make_params(1, H, N, fmt=fmt)

    def call(q, k, v, out, ws, stream):
        qs.qsdpa_forward(q, k, v, out=out, workspace=ws, params=params, stream=stream)

    _replays_match_eager(call, params, f"forward {fmt}",
                         lambda q, k, v: from_dev(qs.qsdpa_forward(q, k, v, params=params)))


def test_noalloc_graph_replays_match_eager(gpu_lib):
    params = qs.make_params(1, H, N, fmt="fp8")

    def call(q, k, v, out, ws, stream):
        qs.qsdpa_forward_noalloc(q, k, v, out, params, stream=stream)

    _replays_match_eager(call, params, "forward_noalloc fp8",
                         lambda q, k, v: from_dev(qs.qsdpa_forward(q, k, v, params=params)))


def test_selective_correction_graph_replays_match_eager(gpu_lib):
    params = qs.make_params(1, H, N, fmt="fp8")
    nbytes = qs.qsdpa_vc_workspace_bytes(params)
    vws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call(q, k, v, out, ws, stream):
        qs.qsdpa_forward_vc(q, k, v, out=out, workspace=vws, params=params, stream=stream)

    _replays_match_eager(call, params, "forward_vc fp8",
                         lambda q, k, v: from_dev(qs.qsdpa_forward_vc(q, k, v, params=params)[0]))
