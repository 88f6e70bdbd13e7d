"""Decode over an FP8 (E4M3) KV pool on the GPU against the fp64 oracle over the dequantized
K/V (O max-abs 1e-2, LSE max-abs 1e-3): local rows at window edges and across many windows,
every split policy, the 12B local geometry, a head_dim 256 global layer, the global family at
head_dim 512 with and without K = V (and its single-KV-head 12B layer), the full local and global
decode batches, poisoned never-visible slots, fail-closed rows, a graph replay, and pools whose
pages sit past byte offset 2^32."""
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


def check(ref, out, lse, tag):
    ref_o, ref_l = ref
    eo = float(np.max(np.abs(out - ref_o)))
    el = float(np.max(np.abs(lse - ref_l)))
    print(f"{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_LSE, (tag, eo, el)


def _local_rows(key, n=14, hi=9000):
    L = workloads.ragged(key, 1, hi, n)
    L[:8] = [1, 15, 16, 17, 1023, 1024, 1025, 2049]
    return L


@pytest.mark.parametrize("split", [512, 1024, 256, 0])
def test_fp8_local_decode(devio, split):
    spec = workloads.LOCAL_31B
    L = _local_rows((81, 1))
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (81, 1), back="visible", poison=True,
                             extra_pages=2)
    workloads.with_fp8_kv(b)
    out, lse = devio.decode_fp8(b, split)
    check(oracle.attend_batch(b), out, lse, f"fp8 local decode split {split}")


def test_fp8_local_decode_12b(devio):
    spec = workloads.LOCAL_12B
    L = _local_rows((81, 2), n=10)
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (81, 2), back="visible", poison=True)
    workloads.with_fp8_kv(b, 0.05, 0.0125)
    out, lse = devio.decode_fp8(b, 512)
    check(oracle.attend_batch(b), out, lse, "fp8 12B local decode")


@pytest.mark.parametrize("split", [512, 0])
def test_fp8_global_family_at_head_dim_256(devio, split):
    """The kernel is family-agnostic: a full-causal layer at head_dim 256, g = 4."""
    spec = workloads.LayerSpec("global", 8, 2, 256)
    L = workloads.ragged((81, 3), 1, 5000, 6)
    L[0] = 1
    b = workloads.make_batch(spec, L, np.ones(6, np.int32), (81, 3), back="visible", poison=True)
    workloads.with_fp8_kv(b)
    out, lse = devio.decode_fp8(b, split)
    check(oracle.attend_batch(b), out, lse, f"fp8 global hd256 split {split}")


def test_fp8_local_decode_full_batch(devio):
    """The local decode workload at full size (64 rows, 512 .. 32768 tokens, split 512)."""
    b = workloads.cfg3_local_decode()
    workloads.with_fp8_kv(b)
    out, lse = devio.decode_fp8(b, 512)
    check(oracle.attend_batch(b), out, lse, "fp8 local decode B=64")


def test_fp8_scales_reach_scores_and_output(devio):
    """Scales changed after the codes were drawn: K codes standing for 4x larger values (sharper
    softmax), V codes for half as large ones. Dropping or swapping a scale moves the LSE and O far
    beyond the tolerance."""
    spec = workloads.LOCAL_31B
    L = np.array([700, 1500, 33], np.int32)
    b = workloads.make_batch(spec, L, np.ones(3, np.int32), (81, 4), back="visible", poison=True)
    workloads.with_fp8_kv(b, 0.025, 0.0213)
    b.fp8.k_scale, b.fp8.v_scale = 0.1, 0.01065
    out, lse = devio.decode_fp8(b, 512)
    check(oracle.attend_batch(b), out, lse, "fp8 rescaled")


def test_fp8_decode_fails_closed(devio):
    """A visible page id out of range in one row turns that row's outputs into NaN; the other rows
    are unaffected."""
    import torch
    spec = workloads.LOCAL_31B
    L = np.array([900, 2000, 40], np.int32)
    b = workloads.make_batch(spec, L, np.ones(3, np.int32), (81, 5), back="visible")
    workloads.with_fp8_kv(b)
    d = devio.DeviceBatch(b)
    pt = b.page_table.copy()
    pt[1, (L[1] - 1) // 16] = b.num_pages
    d.page_table = devio.dev(pt)
    d.decode_fp8(512)
    out, lse = d.result()
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    ref = oracle.attend_batch(b, rows=[0, 2])
    check(ref, out[[0, 2]], lse[[0, 2]], "fp8 fail-closed neighbours")
    torch.cuda.synchronize()


def test_fp8_decode_graph_replay(devio):
    """gattn_decode_fp8kv only enqueues kernels (split kernel and combine), so a capture replays:
    three replays, each after eager work that overwrites every output, reproduce the eager result
    bit for bit, and that matches the oracle."""
    import torch
    spec = workloads.LOCAL_31B
    L = _local_rows((81, 6), n=9)
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (81, 6), back="visible", poison=True)
    workloads.with_fp8_kv(b)
    d = devio.DeviceBatch(b)
    d.decode_fp8(512)  # eager; allocates the workspace before the capture
    eager = d.result()
    check(oracle.attend_batch(b), *eager, "fp8 eager before capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.decode_fp8(512)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        d.decode_fp8(512)
    torch.cuda.synchronize()
    for rep in range(3):
        d.out.fill_(rep + 1)
        d.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, l = d.result()
        assert np.array_equal(o, eager[0]) and np.array_equal(l, eager[1]), rep


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_page_ids_past_4_gib(devio, fp8):
    """The batch's pages moved to ids 70000 and up, i.e. past byte offset 2^32 of their pools
    (about 9.2 GB per bf16 pool, 4.6 GB per FP8 pool): the 64-bit page addressing reads them, and
    the pages below them, all NaN, are never touched."""
    import torch
    spec = workloads.LOCAL_31B
    L = np.array([1, 1025, 3000, 700, 17], np.int32)
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (81, 7), back="visible", poison=True)
    if fp8:
        workloads.with_fp8_kv(b)
    base = 70000
    d = devio.DeviceBatch(b)
    n_pages = base + b.num_pages
    shape = (n_pages, spec.num_kv_heads, spec.page_size, spec.head_dim)
    if fp8:
        assert base * spec.num_kv_heads * spec.page_size * spec.head_dim > 2 ** 32
        for name in ("k_pool8", "v_pool8"):
            big = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
            big[base:] = getattr(d, name)
            setattr(d, name, big)
    else:
        for name in ("k_pool", "v_pool"):
            big = torch.full(shape, int(workloads.BF16_NAN), dtype=torch.int16, device="cuda")
            big[base:] = getattr(d, name)
            setattr(d, name, big)
    d.page_table = devio.dev(np.where(b.page_table >= 0, b.page_table + base, -1).astype(np.int32))
    d.num_pages = n_pages
    if fp8:
        d.decode_fp8(512)
    else:
        d.decode(512)
    out, lse = d.result()
    check(oracle.attend_batch(b), out, lse, f"{'fp8' if fp8 else 'bf16'} pages past 4 GiB")
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("spec,split", [(workloads.GLOBAL_31B, 512), (workloads.GLOBAL_31B, 0),
                                        (workloads.GLOBAL_31B_KV_SHARED, 1024), (workloads.GLOBAL_31B_KV_SHARED, 512),
                                        (workloads.GLOBAL_12B, 512)],
                         ids=["global-512", "global-unsplit", "kv-shared-1024", "kv-shared-512", "12b-global"])
def test_fp8_global_decode(devio, spec, split):
    """The global family over E4M3 pools (head_dim 512; with K = V the V side is the K codes with
    the K scale): ragged rows from 1 token across split edges, poisoned slots."""
    L = workloads.ragged((82, spec.num_kv_heads, int(spec.kv_shared)), 1, 6000, 8)
    L[:4] = [1, 16, 1024, 1025]
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (82, int(spec.kv_shared)), back="visible",
                             poison=True)
    workloads.with_fp8_kv(b)
    out, lse = devio.decode_fp8(b, split)
    check(oracle.attend_batch(b), out, lse, f"fp8 {spec.num_kv_heads}-head global K=V={spec.kv_shared} split {split}")


def test_fp8_global_decode_full_batch(devio):
    """The 32-row global decode workload (contexts ~U{1..8192}, split 512) over E4M3 pools."""
    b = workloads.cfg2_global_decode()
    workloads.with_fp8_kv(b)
    out, lse = devio.decode_fp8(b, 512)
    check(oracle.attend_batch(b), out, lse, "fp8 global decode B=32")
