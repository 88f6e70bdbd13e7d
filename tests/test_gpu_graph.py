"""HIP graph capture of the library's calls (the launch discipline of a serving step).

gattn_decode and gattn_prefill only enqueue kernels on the caller's stream: no allocation, no
memset, no synchronisation, with per-row lengths read on the device. So a step of several layers
can be captured once and replayed. Six decode layers in the sweep's order (five local, then one
global with K = V) and one prefill of each family are captured in one graph; three replays, each
after eager work that overwrites every output, must reproduce the eager results bit for bit, and
those match the fp64 oracle.
"""
import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


@pytest.fixture(scope="module")
def devio():
    import torch
    assert torch.cuda.is_available()
    from global_paged_gqa_amd import devio as d
    return d


def test_graph_replays_match_eager(devio):
    import torch
    specs = [workloads.LOCAL_31B] * 5 + [workloads.GLOBAL_31B_KV_SHARED]
    calls = []
    batches = []
    for l, spec in enumerate(specs):
        L = workloads.ragged((7, l), 1, 6000, 6)
        b = workloads.make_batch(spec, L, np.ones(6, np.int32), (7, l), back="visible", poison=True)
        calls.append((devio.DeviceBatch(b), "decode", 1024 if spec.is_global else 512))
        batches.append(b)
    for f, spec in enumerate((workloads.GLOBAL_31B, workloads.LOCAL_31B)):
        b = workloads.make_batch(spec, [700, 1300], [200, 300], (7, 10 + f), back="visible", poison=True)
        calls.append((devio.DeviceBatch(b), "prefill", None))
        batches.append(b)

    def step():
        for d, kind, split in calls:
            if kind == "decode":
                d.decode(split)
            else:
                d.prefill()

    step()  # eager; also allocates every workspace before the capture
    torch.cuda.synchronize()
    eager = [d.result() for d, _, _ in calls]
    for b, (o, l) in zip(batches, eager):
        ref_o, ref_l = oracle.attend_batch(b)
        assert np.max(np.abs(o - ref_o)) <= TOL_O and np.max(np.abs(l - ref_l)) <= TOL_LSE

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for d, _, _ in calls:  # eager work between replays: every output overwritten
            d.out.fill_(rep + 1)
            d.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (d, _, _) in enumerate(calls):
            o, l = d.result()
            assert np.array_equal(o, eager[i][0]) and np.array_equal(l, eager[i][1]), (rep, i)
