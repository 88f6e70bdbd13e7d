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


def _run(devio, spec, b, L, n_new, cu, k_new, v_new, page_table=None, max_new=None):
    import torch
    nat = devio.nat
    lay = devio.layer_of(spec)
    kp = devio.dev(b.k_pool)
    vp = None if b.v_pool is None else devio.dev(b.v_pool)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pt = b.page_table if page_table is None else page_table
    nat.gattn_kv_append(lay, devio.dev(k_new), None if v_new is None else devio.dev(v_new), kp, vp, b.num_pages,
                        devio.dev(pt.astype(np.int32)), pt.shape[1], devio.dev(cu), devio.dev(L), b.B,
                        int(n_new.max()) if max_new is None else int(max_new), status)
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


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.LOCAL_31B], ids=["global", "local"])
def test_kv_append_fails_closed(devio, spec):
    """Out-of-range and -1 page ids, positions beyond the table and rows with more new tokens
    than cached ones write nothing and raise the status flag; every other token is written. (At
    head_dim 256 the kernel reads a token's source row before its page id, at 512 after: both
    orders are covered.)"""
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
def test_kv_append_row_above_max_new_fails_closed(devio, spec):
    """max_new (the host bound that sizes the grid) below one row's count of new tokens: that row
    (2048 new tokens against the largest count of the others, 300 or less) writes none of them and
    raises the status flag, where a fail-open kernel would write the tokens its grid covers and
    silently drop the rest; every other row is written as usual."""
    b, L, n_new, cu, k_new, v_new = _case(spec, (44, spec.num_kv_heads))
    mx = int(n_new[1:].max())
    assert n_new[0] == 2048 and 0 < mx < 2048
    kp, vp, status = _run(devio, spec, b, L, n_new, cu, k_new, v_new, max_new=mx)
    ref_k, ref_v, skipped = oracle.kv_append(spec.num_kv_heads, spec.head_dim, spec.page_size, cu, L, b.page_table,
                                             b.num_pages, k_new, v_new, b.k_pool, b.v_pool, max_new=mx)
    assert skipped == 2048 and status == 1
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


# ---------------------------------------------------------------- FP8 (E4M3) pools
def _run_fp8(devio, spec, b, L, n_new, cu, k_new, v_new, k8, v8, ks, vs, page_table=None):
    import torch
    nat = devio.nat
    kp = torch.from_numpy(np.ascontiguousarray(k8)).to("cuda")
    vp = torch.from_numpy(np.ascontiguousarray(v8)).to("cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pt = b.page_table if page_table is None else page_table
    nat.gattn_kv_append_fp8(devio.layer_of(spec), devio.dev(k_new), devio.dev(v_new), kp, vp, ks, vs, b.num_pages,
                            devio.dev(pt.astype(np.int32)), pt.shape[1], devio.dev(cu), devio.dev(L), b.B,
                            int(n_new.max()), status)
    torch.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("ks,vs", [(0.5, 2.0 ** -7), (0.0371, 0.0213)], ids=["dyadic", "non-dyadic"])
def test_kv_append_fp8_every_bf16_value(devio, ks, vs):
    """All 65536 bf16 bit patterns (NaN, infinities, subnormals, exact midpoints under the dyadic
    scales) appended into E4M3 pools: every byte equals the oracle's encoder output."""
    spec = workloads.LOCAL_31B
    Hkv, hd = spec.num_kv_heads, spec.head_dim
    T = 65536 // (Hkv * hd)                   # 16 tokens hold every pattern once
    L = np.array([T + 5, 1], np.int32)
    n_new = np.array([T, 0], np.int32)
    cu = np.array([0, T, T], np.int32)
    b = workloads.make_batch(spec, L, np.ones(2, np.int32), (44, 0), back="all", extra_pages=1)
    k_new = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, hd)
    v_new = np.ascontiguousarray(k_new[::-1])
    g = np.random.default_rng(44)
    k8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    v8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    kp, vp, status = _run_fp8(devio, spec, b, L, n_new, cu, k_new, v_new, k8, v8, ks, vs)
    ref_k, ref_v, skipped = oracle.kv_append_fp8(Hkv, hd, spec.page_size, cu, L, b.page_table, b.num_pages, k_new,
                                                 v_new, ks, vs, k8, v8)
    assert skipped == 0 and status == 0
    assert np.array_equal(kp, ref_k) and np.array_equal(vp, ref_v)


@pytest.mark.parametrize("spec", [workloads.LOCAL_31B, workloads.LOCAL_12B], ids=["31b", "12b"])
def test_kv_append_fp8_bitwise_and_fails_closed(devio, spec):
    """Ragged rows (0, 1, a page, page-crossing, a 2048-token chunk), a bad page id and a row with
    more new tokens than cached ones: bytes equal the oracle's, the status flag rises."""
    b, L, n_new, cu, k_new, v_new = _case(spec, (45, spec.num_kv_heads))
    pt = b.page_table.copy()
    pt[3, (L[3] - 1) // 16] = -1
    L_bad = L.copy()
    L_bad[4] = 3
    g = np.random.default_rng(45)
    k8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    v8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    ks, vs = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE
    kp, vp, status = _run_fp8(devio, spec, b, L_bad, n_new, cu, k_new, v_new, k8, v8, ks, vs, page_table=pt)
    ref_k, ref_v, skipped = oracle.kv_append_fp8(spec.num_kv_heads, spec.head_dim, spec.page_size, cu, L_bad, pt,
                                                 b.num_pages, k_new, v_new, ks, vs, k8, v8)
    assert skipped > 0 and status == 1
    assert np.array_equal(kp, ref_k) and np.array_equal(vp, ref_v)


def test_append_fp8_then_decode_fp8(devio):
    """Decode rows whose last tokens were just appended into NaN-filled E4M3 slots: the decode over
    the pool the append built matches the oracle over the oracle-appended codes."""
    import torch
    spec = workloads.LOCAL_31B
    L = np.array([1, 17, 1024, 1500, 3000], np.int32)
    C = np.array([1, 17, 300, 1, 64], np.int32)
    b = workloads.make_batch(spec, L, np.ones(5, np.int32), (46, 1), back="visible")
    workloads.with_fp8_kv(b)
    f = b.fp8
    cu = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    k_new, v_new = [], []
    for r in range(b.B):
        kk, vv = b.row_keys(r)
        k_new.append(kk[len(kk) - C[r]:])
        v_new.append(vv[len(vv) - C[r]:])
    k_new, v_new = np.concatenate(k_new), np.concatenate(v_new)
    k8, v8 = f.k_pool.copy(), f.v_pool.copy()
    for r in range(b.B):  # the appended slots hold NaN codes before the append
        for t in range(L[r] - C[r], L[r]):
            k8[b.page_table[r, t // 16], :, t % 16, :] = 0x7F
            v8[b.page_table[r, t // 16], :, t % 16, :] = 0xFF
    ref_k, ref_v, skipped = oracle.kv_append_fp8(spec.num_kv_heads, spec.head_dim, 16, cu, L, b.page_table,
                                                 b.num_pages, k_new, v_new, f.k_scale, f.v_scale, k8, v8)
    assert skipped == 0
    d = devio.DeviceBatch(b)
    d.k_pool8 = torch.from_numpy(k8).to("cuda")
    d.v_pool8 = torch.from_numpy(v8).to("cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    devio.nat.gattn_kv_append_fp8(d.layer, devio.dev(k_new), devio.dev(v_new), d.k_pool8, d.v_pool8, f.k_scale,
                                  f.v_scale, b.num_pages, d.page_table, b.pt_stride, devio.dev(cu), d.ctx_lens, b.B,
                                  int(C.max()), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(d.k_pool8.cpu().numpy(), ref_k) and np.array_equal(d.v_pool8.cpu().numpy(), ref_v)
    d.decode_fp8(512)
    out, lse = d.result()
    # the oracle side: the contiguous rows re-gathered from the oracle-appended pools
    P = 16
    ks8, vs8 = [], []
    for r in range(b.B):
        toks = np.arange(int(b.k_starts[r]), int(L[r]))
        ks8.append(ref_k[b.page_table[r, toks // P], :, toks % P, :])
        vs8.append(ref_v[b.page_table[r, toks // P], :, toks % P, :])
    ref_o, ref_l = oracle.attend_fp8kv(False, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.window,
                                       spec.softmax_scale, b.q_lens, b.ctx_lens, b.k_starts, b.q,
                                       np.concatenate(ks8), np.concatenate(vs8), f.k_scale, f.v_scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(out - ref_o)) <= 1e-2 and np.max(np.abs(lse - ref_l)) <= 1e-3


def test_append_and_prefill_past_4_gib(devio):
    """Page ids from 70000 up (past byte offset 2^32 of each bf16 pool): the append writes the
    chunk's K/V there and the prefill reads them back; the pages below stay NaN and untouched."""
    import torch
    spec = workloads.LOCAL_31B
    L = np.array([700, 1500], np.int32)
    C = np.array([200, 300], np.int32)
    b = workloads.make_batch(spec, L, C, (47, 1), back="visible")
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
    base = 70000
    d = devio.DeviceBatch(b)
    n_pages = base + b.num_pages
    shape = (n_pages, spec.num_kv_heads, spec.page_size, spec.head_dim)
    for name in ("k_pool", "v_pool"):
        big = torch.full(shape, int(workloads.BF16_NAN), dtype=torch.int16, device="cuda")
        big[base:] = getattr(d, name)
        setattr(d, name, big)
    d.page_table = devio.dev(np.where(b.page_table >= 0, b.page_table + base, -1).astype(np.int32))
    d.num_pages = n_pages
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    devio.nat.gattn_kv_append(d.layer, devio.dev(k_new), devio.dev(v_new), d.k_pool, d.v_pool, n_pages, d.page_table,
                              b.pt_stride, devio.dev(cu), d.ctx_lens, b.B, int(C.max()), status)
    d.prefill()
    out, lse = d.result()
    assert int(status.item()) == 0
    low = d.k_pool[:base].view(-1)
    assert bool((low == int(workloads.BF16_NAN)).all())
    ref_o, ref_l = oracle.attend_batch(b)
    assert np.max(np.abs(out - ref_o)) <= 1e-2 and np.max(np.abs(lse - ref_l)) <= 1e-3
    del d, low
    torch.cuda.empty_cache()


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.GLOBAL_31B_KV_SHARED], ids=["global", "kv-shared"])
def test_kv_append_fp8_global_bitwise(devio, spec):
    """E4M3 append at head_dim 512 (with K = V only the K pool is written): bytes equal the oracle's."""
    import torch
    b, L, n_new, cu, k_new, v_new = _case(spec, (48, int(spec.kv_shared)))
    g = np.random.default_rng(48)
    k8 = g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    v8 = None if spec.kv_shared else g.integers(0, 256, size=b.k_pool.shape, dtype=np.uint8)
    ks, vs = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE
    kp = torch.from_numpy(k8).to("cuda")
    vp = None if v8 is None else torch.from_numpy(v8).to("cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    devio.nat.gattn_kv_append_fp8(devio.layer_of(spec), devio.dev(k_new), None if v_new is None else devio.dev(v_new),
                                  kp, vp, ks, vs, b.num_pages, devio.dev(b.page_table.astype(np.int32)), b.pt_stride,
                                  devio.dev(cu), devio.dev(L), b.B, int(n_new.max()), status)
    torch.cuda.synchronize()
    ref_k, ref_v, skipped = oracle.kv_append_fp8(spec.num_kv_heads, spec.head_dim, spec.page_size, cu, L, b.page_table,
                                                 b.num_pages, k_new, v_new, ks, vs, k8, v8)
    assert skipped == 0 and int(status.item()) == 0
    assert np.array_equal(kp.cpu().numpy(), ref_k)
    if vp is not None:
        assert np.array_equal(vp.cpu().numpy(), ref_v)
