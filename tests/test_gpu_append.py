"""KV append on the GPU: bit-exact against the oracle's scatter, fail-closed on bad page ids, and
end to end (append a chunk's K/V into poisoned slots, then attend over them)."""
import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

SPECS = [workloads.GLOBAL_31B, workloads.LOCAL_31B, workloads.GLOBAL_31B_KV_SHARED, workloads.GLOBAL_12B]
IDS = ["global", "local", "kv-shared", "12b-global"]


@pytest.fixture(scope="module")
def devio():
    import torch
    assert torch.cuda.is_available()
    from global_paged_gqa_amd import devio as d
    return d


def _case(spec, key, B=7, max_len=5000):
    """Rows with random lengths and random numbers of new tokens (0, 1, a page, page-crossing,
    a whole 2048-token chunk), a globally shuffled table, pools of bf16 NaN except the slots
    already written, and the new tokens' K/V rows."""
    g = workloads.generator(*key, 0)
    L = g.integers(1, max_len, size=B).astype(np.int32)
    L[0], L[1] = 2048, 17
    n_new = np.minimum(L, np.array([2048, 17, 0, 1, 16, 33, 300][:B], np.int32))
    b = workloads.make_batch(spec, L, np.ones(B, np.int32), key, back="all", poison=True, extra_pages=3)
    b.k_pool[:] = workloads.BF16_NAN
    if b.v_pool is not None:
        b.v_pool[:] = workloads.BF16_NAN
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    T = int(cu[-1])
    k_new = workloads.normal_bf16(workloads.generator(*key, 1), (T, spec.num_kv_heads, spec.head_dim))
    v_new = None if spec.kv_shared else workloads.normal_bf16(workloads.generator(*key, 2),
                                                               (T, spec.num_kv_heads, spec.head_dim))
    return b, L, n_new, cu, k_new, v_new


def _run(devio, spec, b, L, n_new, cu, k_new, v_new, page_table=None):
    import torch
    nat = devio.nat
    lay = devio.layer_of(spec)
    kp = devio.dev(b.k_pool)
    vp = None if b.v_pool is None else devio.dev(b.v_pool)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pt = b.page_table if page_table is None else page_table
    nat.gattn_kv_append(lay, devio.dev(k_new), None if v_new is None else devio.dev(v_new), kp, vp, b.num_pages,
                        devio.dev(pt.astype(np.int32)), pt.shape[1], devio.dev(cu), devio.dev(L), b.B,
                        int(n_new.max()), status)
    torch.cuda.synchronize()
    kp_h = kp.cpu().numpy().view(np.uint16)
    vp_h = None if vp is None else vp.cpu().numpy().view(np.uint16)
    return kp_h, vp_h, int(status.item())


@pytest.mark.parametrize("spec", SPECS, ids=IDS)
def test_kv_append_bitwise(devio, spec):
    b, L, n_new, cu, k_new, v_new = _case(spec, (41, spec.num_kv_heads, int(spec.kv_shared), spec.num_q_heads))
    kp, vp, status = _run(devio, spec, b, L, n_new, cu, k_new, v_new)
    ref_k, ref_v, skipped = oracle.kv_append(spec.num_kv_heads, spec.head_dim, spec.page_size, cu, L, b.page_table,
                                             b.num_pages, k_new, v_new, b.k_pool, b.v_pool)
    assert skipped == 0 and status == 0
    assert np.array_equal(kp, ref_k)
    if v_new is not None:
        assert np.array_equal(vp, ref_v)


def test_kv_append_fails_closed(devio):
    """Out-of-range and -1 page ids, positions beyond the table and rows with more new tokens
    than cached ones write nothing and raise the status flag; every other token is written."""
    spec = workloads.GLOBAL_31B
    b, L, n_new, cu, k_new, v_new = _case(spec, (42, 0))
    pt = b.page_table.copy()
    pt[2, 0] = b.num_pages + 5           # row 2 has no new tokens: never read, no flag from it
    pt[3, (L[3] - 1) // 16] = -1         # row 3's single new token: unbacked page
    pt[5, (L[5] - 1) // 16] = b.num_pages  # row 5: its last page out of range
    L_bad = L.copy()
    L_bad[4] = 3                         # row 4: 16 new tokens but only 3 cached
    kp, vp, status = _run(devio, spec, b, L_bad, n_new, cu, k_new, v_new, page_table=pt)
    ref_k, ref_v, skipped = oracle.kv_append(spec.num_kv_heads, spec.head_dim, spec.page_size, cu, L_bad, pt,
                                             b.num_pages, k_new, v_new, b.k_pool, b.v_pool)
    assert skipped > 0 and status == 1
    assert np.array_equal(kp, ref_k) and np.array_equal(vp, ref_v)


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.LOCAL_31B], ids=["global", "local"])
def test_append_then_prefill(devio, spec):
    """A chunk's K/V appended into slots that held NaN, then the chunk's prefill: the outputs match
    the oracle on the contiguous K/V (the cache the append built is the one attention reads)."""
    import torch
    L = np.array([700, 1500], np.int32)
    C = np.array([200, 1100], np.int32)
    b = workloads.make_batch(spec, L, C, (43, spec.num_kv_heads), back="all")
    cu = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    k_new, v_new = [], []
    for r in range(b.B):
        kk, vv = b.row_keys(r)
        k_new.append(kk[len(kk) - C[r]:])
        v_new.append(vv[len(vv) - C[r]:])
    k_new, v_new = np.concatenate(k_new), np.concatenate(v_new)
    for r in range(b.B):  # the chunk's slots hold NaN before the append
        for t in range(L[r] - C[r], L[r]):
            b.k_pool[b.page_table[r, t // 16], :, t % 16, :] = workloads.BF16_NAN
            b.v_pool[b.page_table[r, t // 16], :, t % 16, :] = workloads.BF16_NAN
    d = devio.DeviceBatch(b)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    devio.nat.gattn_kv_append(d.layer, devio.dev(k_new), devio.dev(v_new), d.k_pool, d.v_pool, b.num_pages,
                              d.page_table, b.pt_stride, devio.dev(cu), d.ctx_lens, b.B, int(C.max()), status)
    d.prefill()
    out, lse = d.result()
    ref_o, ref_l = oracle.attend_batch(b)
    assert int(status.item()) == 0
    assert np.max(np.abs(out - ref_o)) <= 1e-2 and np.max(np.abs(lse - ref_l)) <= 1e-3
