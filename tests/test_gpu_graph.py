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


@pytest.mark.parametrize("spec,split", [(workloads.GLOBAL_31B, 512), (workloads.GLOBAL_31B_KV_SHARED, 1024),
                                        (workloads.LOCAL_31B, 512)], ids=["global", "global-kv-shared", "local"])
def test_decode_graph_bucket_set(devio, spec, split):
    """A bucket set {1, 4, 8, 16} captured over one fixed 16-row batch. For batches of 1, 3, 8, 11
    and 16 rows the serving loop sets the lengths of the rows past the batch to 0 and replays the
    smallest bucket that holds it, three times, each after eager work that overwrites the outputs.
    The batch's rows equal gattn_decode over those rows alone, bit for bit, on every replay; the
    padding rows inside the bucket fail closed (NaN), the rows past it are not written."""
    import torch
    from global_paged_gqa_amd import _native as nat
    B, max_ctx, buckets = 16, 8192, [1, 4, 8, 16]
    L = workloads.ragged((31, int(spec.kv_shared), int(spec.is_global)), 1, 6000, B)
    b = workloads.make_batch(spec, L, np.ones(B, np.int32), (31, int(spec.kv_shared), int(spec.is_global)),
                             back="visible", poison=True, pt_stride=max_ctx // 16)
    d = devio.DeviceBatch(b)
    need = nat.gattn_decode_workspace_bytes(d.layer, B, max_ctx, split)
    ws = torch.full((max(need, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    h = nat.gattn_decode_graphs_create(d.layer, d.q, d.k_pool, d.v_pool, d.num_pages, d.page_table, d.pt_stride,
                                       d.ctx_lens, max_ctx, split, ws, need, d.out, d.lse, buckets)
    try:
        for n in (1, 3, 8, 11, 16):
            bucket = nat.gattn_decode_graphs_bucket(h, n)
            assert bucket == min(x for x in buckets if x >= n)
            ref = devio.DeviceBatch(b.subset(range(n)))
            ref.decode(split, max_ctx)
            ref_o, ref_l = ref.result()
            lens = np.asarray(L, np.int32).copy()
            lens[n:] = 0
            d.ctx_lens.copy_(torch.from_numpy(lens).to("cuda"))
            for rep in range(3):
                d.out.fill_(7)              # eager work between the replays
                d.lse.fill_(-3.0)
                torch.cuda.synchronize()
                nat.gattn_decode_graphs_launch(h, n)
                o, l = d.result()
                assert np.array_equal(o[:n], ref_o) and np.array_equal(l[:n], ref_l), (n, rep)
                assert np.all(np.isnan(l[n:bucket])) and np.all(np.isnan(o[n:bucket])), (n, rep)
                assert np.all(l[bucket:] == -3.0), (n, rep)
        with pytest.raises(nat.GattnError) as e:
            nat.gattn_decode_graphs_launch(h, B + 1)
        assert e.value.status == nat.ERR_BAD_SHAPE
    finally:
        torch.cuda.synchronize()
        nat.gattn_decode_graphs_destroy(h)
