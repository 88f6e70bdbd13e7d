"""Split-KV decode on the GPU against the fp64 oracle, plus the bitwise invariances.

Tolerances: O max-abs 1e-2, fp32 LSE max-abs 1e-3 on unit-normal bf16 inputs;
page-table and index handling bit-exact (probes, invariance under page
placement, batch composition and row order).
"""
import math

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


def check(batch, out, lse, rows=None, tag="", bf16_slack=False):
    """O within 1e-2 and LSE within 1e-3 of the oracle. With bf16_slack (only for scales sharper
    than 1/sqrt(hd), where |O| can exceed 2.5) the O bar also admits the output format's own
    rounding, half a bf16 ulp of the reference value (2^-9 |O|)."""
    ref_o, ref_l = oracle.attend_batch(batch, rows)
    if rows is not None:
        cq = batch.cu_q
        idx = np.concatenate([np.arange(cq[r], cq[r + 1]) for r in rows])
        out, lse = out[idx], lse[idx]
    err = np.abs(out - ref_o)
    if bf16_slack:
        err = err - np.abs(ref_o) * 2.0 ** -9
    eo = float(np.max(err)) if out.size else 0.0
    el = float(np.max(np.abs(lse - ref_l))) if lse.size else 0.0
    print(f"{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


@pytest.mark.parametrize("split", [0, 16, 512, 1024])
def test_cfg1_tiny_local_decode(devio, split):
    b = workloads.cfg1_tiny_decode()
    out, lse = devio.decode(b, split)
    check(b, out, lse, tag=f"cfg1 S={split}")


@pytest.mark.parametrize("split", [0, 16, 512])
def test_global_decode_small(devio, split):
    b = workloads.cfg2_global_decode(B=6, max_len=1500)
    out, lse = devio.decode(b, split)
    check(b, out, lse, tag=f"global small S={split}")


def test_cfg2_global_decode_full(devio):
    b = workloads.cfg2_global_decode()
    out, lse = devio.decode(b, 512)
    check(b, out, lse, tag="cfg2 full")


@pytest.mark.parametrize("split", [0, 512, 1024])
def test_local_decode_small(devio, split):
    b = workloads.cfg3_local_decode(B=6, lo=1, hi=5000)
    out, lse = devio.decode(b, split)
    check(b, out, lse, tag=f"local small S={split}")


@pytest.mark.parametrize("split", [512, 256])
def test_local_rows_ending_on_a_split_boundary(devio, split):
    """Local rows whose context ends exactly on a split boundary, in a page table exactly as wide
    as the longest row: a row's last split slot is then empty and starts past the row's last table
    entry (the workgroup that merges a row's slots must not read that entry), beside rows whose
    windows are cut by the splits elsewhere."""
    L = np.array([2048, 1536, 2048, 1000, 2048], np.int32)
    b = workloads.make_batch(workloads.LOCAL_31B, L, np.ones(len(L), np.int32), (61, split), back="all")
    assert b.pt_stride == 2048 // 16
    out, lse = devio.decode(b, split)
    check(b, out, lse, tag=f"split-boundary rows S={split}")


def test_cfg3_local_decode_full(devio):
    b = workloads.cfg3_local_decode()
    out, lse = devio.decode(b, 512)
    check(b, out, lse, tag="cfg3 full")


@pytest.mark.parametrize("split", [0, 64, 1024])
def test_global_kv_shared_decode(devio, split):
    spec = workloads.GLOBAL_31B_KV_SHARED
    L = workloads.ragged((5, 9), 1, 3000, 5)
    b = workloads.make_batch(spec, L, np.ones(5, np.int32), (5, 9), back="all")
    out, lse = devio.decode(b, split)
    check(b, out, lse, tag=f"global K=V S={split}")


@pytest.mark.parametrize("fam,hkv,hd", [("local", 1, 256), ("global", 2, 512), ("global", 4, 256),
                                        ("local", 8, 512)])
@pytest.mark.parametrize("g", [1, 3, 16])
def test_group_sizes_and_head_dims(devio, fam, hkv, hd, g):
    spec = workloads.LayerSpec(fam, hkv * g, hkv, hd, window=300 if fam == "local" else 0, scale=1.0 / 3.0)
    L = workloads.ragged((6, g, hd), 1, 900, 3)
    b = workloads.make_batch(spec, L, np.ones(3, np.int32), (6, g, hd, hkv), back="visible")
    out, lse = devio.decode(b, 128)
    check(b, out, lse, tag=f"{fam} hkv={hkv} g={g} hd={hd}", bf16_slack=True)


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 1023, 1024, 1025, 2048, 2049, 3073, 4097])
def test_window_edges(devio, L):
    """Sliding-window boundaries 1023/1024/1025 and multi-window continuation, at split 512."""
    spec = workloads.LayerSpec("local", 4, 2, 256, window=1024)
    b = workloads.make_batch(spec, [L], [1], (7, L), back="visible", poison=True)
    out, lse = devio.decode(b, 512)
    check(b, out, lse, tag=f"window L={L}")


def test_scale_one_variant(devio):
    """Gemma 4's scale = 1.0 convention (hd 512, block-GQA over 4 KV heads)."""
    spec = workloads.LayerSpec("global", 32, 4, 512, scale=1.0)
    L = workloads.ragged((8, 0), 1, 2000, 4)
    b = workloads.make_batch(spec, L, np.ones(4, np.int32), (8, 0), back="all")
    out, lse = devio.decode(b, 512)
    check(b, out, lse, tag="scale 1.0")


# ------------------------------------------------------------------------ bitwise invariances
def _run(devio, b, split, max_ctx=None):
    d = devio.DeviceBatch(b)
    d.decode(split, max_ctx)
    return d.result()


def test_bitwise_invariance_page_placement_poison_and_repeat(devio):
    b = workloads.cfg2_global_decode(B=8, max_len=3000)
    o1, l1 = _run(devio, b, 512)
    o2, l2 = _run(devio, b, 512)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "not deterministic"
    for key in ((11, 1), (11, 2)):
        bp = workloads.permute_pages(b, key, extra_pages=7, fill=int(workloads.BF16_NAN))
        o3, l3 = _run(devio, bp, 512)
        assert np.array_equal(o1, o3) and np.array_equal(l1, l3), key
    bn = workloads.make_batch(b.spec, b.ctx_lens, b.q_lens, b.meta["key"], back="all", poison=True,
                              extra_pages=5)
    o4, l4 = _run(devio, bn, 512)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4), "NaN poison leaked"
    # identity page table
    bi = workloads.make_batch(b.spec, b.ctx_lens, b.q_lens, b.meta["key"], back="all", shuffle=False)
    o5, l5 = _run(devio, bi, 512)
    assert np.array_equal(o1, o5) and np.array_equal(l1, l5)


def test_bitwise_batch_invariance_and_reorder(devio):
    b = workloads.cfg3_local_decode(B=10, lo=1, hi=6000, pt_stride=2048)
    o_all, l_all = _run(devio, b, 512, max_ctx=8192)
    for rows in ([3], [7, 1], [9, 0, 4, 2]):
        sub = workloads.Batch(b.spec, b.ctx_lens[rows], b.q_lens[rows], b.k_starts[rows], b.q[rows], b.k, b.v,
                              b.page_table[rows], b.k_pool, b.v_pool)
        o, l = _run(devio, sub, 512, max_ctx=8192)
        assert np.array_equal(o, o_all[rows]) and np.array_equal(l, l_all[rows]), rows
    # a different grid bound (max_ctx) does not change any row either
    o, l = _run(devio, b, 512, max_ctx=32768)
    assert np.array_equal(o, o_all) and np.array_equal(l, l_all)


@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.GLOBAL_31B_KV_SHARED], ids=["global", "global-kv-shared"])
def test_bitwise_launch_shape_invariance(devio, spec):
    """A head_dim 512 grid of at most 256 (row, KV head, split) items runs a split's page streams
    on one wave each (four with K = V, two with separate pools); up to 512 items on two waves; a
    larger grid on one wave that runs the streams in turn. A row gives the same bits in every shape:
    alone, in 2- and 4-row batches (16 x 4 x 4 = 256 items at most), in a 6-row batch (384 items)
    and inside a 10-row batch (640 items). The small-grid results also match the oracle."""
    L = workloads.ragged((14, int(spec.kv_shared)), 1, 8192, 10)
    L[0], L[1], L[2] = 8192, 1, 513
    b = workloads.make_batch(spec, L, np.ones(10, np.int32), (14, int(spec.kv_shared)), back="all")
    o_all, l_all = _run(devio, b, 512, max_ctx=8192)
    for rows in ([0], [2, 5], [1, 3, 4, 0], [9, 8, 7, 6, 5, 4]):
        sub = b.subset(rows)
        o, l = _run(devio, sub, 512, max_ctx=8192)
        assert np.array_equal(o, o_all[rows]) and np.array_equal(l, l_all[rows]), rows
    check(sub, o, l, tag=f"{spec.family} kv_shared={spec.kv_shared} small grid")



@pytest.mark.parametrize("spec", [workloads.GLOBAL_31B, workloads.GLOBAL_31B_KV_SHARED], ids=["global", "global-kv-shared"])
def test_page_stream_edges(devio, spec):
    """Splits of 128 keys (eight pages) with every page count from one to eight in the last split,
    so that page streams are empty or one page short (four streams with K = V, two with separate
    pools), and a poisoned (NaN) pool behind every unused slot. Each row alone runs the four-wave
    shape with K = V and the two-wave shape otherwise (256 items), two rows the two-wave shape, all
    thirteen the one-wave shape; every row gives the same bits in every shape and matches the
    oracle."""
    L = np.array([1, 16, 17, 33, 49, 64, 65, 90, 100, 113, 128, 8192 - 7, 8192], np.int32)
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), (17, int(spec.kv_shared)), back="all", poison=True)
    o_all, l_all = _run(devio, b, 128, max_ctx=8192)
    check(b, o_all, l_all, tag=f"{spec.family} kv_shared={spec.kv_shared} stream edges")
    for rows in ([0], [4], [7], [12], [2, 9], [11, 5]):
        o, l = _run(devio, b.subset(rows), 128, max_ctx=8192)
        assert np.array_equal(o, o_all[rows]) and np.array_equal(l, l_all[rows]), rows


# ------------------------------------------------------------------------ index probes
def test_count_probe(devio):
    """K = 0: every visible key has weight 1/n, so exp(LSE) is exactly the visible count."""
    for spec in (workloads.LOCAL_31B, workloads.GLOBAL_31B):
        L = workloads.ragged((12, spec.head_dim), 1, 4000, 12)
        b = workloads.make_batch(spec, L, np.ones(12, np.int32), (12, spec.head_dim), back="visible")
        b.k_pool[:] = 0
        out, lse = devio.decode(b, 512)
        n = np.minimum(L, spec.window) if not spec.is_global else L
        assert np.array_equal(np.round(np.exp(lse)).astype(np.int64), np.repeat(n[:, None], spec.num_q_heads, 1))


def test_position_probe(devio):
    """One key dominates: with K[t*] aligned to q and large, every other weight underflows and O
    equals V[t*] bit for bit. Sweeps t* over page, split and window edges."""
    spec = workloads.LayerSpec("local", 4, 2, 256, window=1024, scale=1.0)
    L = 3000
    lo = L - 1024
    for t_star in (lo, lo + 1, lo + 15, 2047, 2048, 2559, 2560, L - 17, L - 16, L - 1):
        b = workloads.make_batch(spec, [L], [1], (13, t_star), back="visible")
        off = t_star - int(b.k_starts[0])
        b.q[:] = 0
        b.q[0, :, 0] = workloads.f32_to_bf16_bits(np.float32([1.0]))[0]
        kk = np.zeros_like(b.k)
        kk[off, :, 0] = workloads.f32_to_bf16_bits(np.float32([200.0]))[0]
        pt = b.page_table[0]
        # rewrite the pool from the contiguous copy (K) and a position code in V
        P = spec.page_size
        code = workloads.f32_to_bf16_bits(np.float32(np.arange(256) + 0.5 + (t_star % 97)))
        vv = b.v.copy()
        vv[off, :, :] = code
        for t in range(int(b.k_starts[0]), L):
            b.k_pool[pt[t // P], :, t % P, :] = kk[t - int(b.k_starts[0])]
            b.v_pool[pt[t // P], :, t % P, :] = vv[t - int(b.k_starts[0])]
        out, _ = devio.decode(b, 512)
        want = workloads.bf16_bits_to_f32(code).astype(np.float64)
        for h in range(4):
            assert np.array_equal(out[0, h], want), t_star


# ------------------------------------------------------------------------ fail closed on device
def test_bad_lengths_and_pages_give_nan_rows_only(devio):
    import torch
    b = workloads.cfg2_global_decode(B=4, max_len=900, pt_stride=64)
    d = devio.DeviceBatch(b)
    d.decode(512, max_ctx=1024)
    good_o, good_l = d.result()
    cl = b.ctx_lens.copy()
    cl[1] = 2000                     # beyond max_ctx
    d.ctx_lens.copy_(torch.from_numpy(cl).cuda())
    pt = b.page_table.copy()
    pt[2, (b.ctx_lens[2] - 1) // 16] = b.num_pages + 5   # a visible page out of range
    d.page_table.copy_(torch.from_numpy(pt).cuda())
    d.decode(512, max_ctx=1024)
    o, l = d.result()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(l[1]))
    assert np.all(np.isnan(o[2])) and np.all(np.isnan(l[2]))
    for r in (0, 3):
        assert np.array_equal(o[r], good_o[r]) and np.array_equal(l[r], good_l[r])


# ------------------------------------------------------------------------ exported combine
@pytest.mark.parametrize("hd,ns", [(512, 7), (256, 3), (1024, 40), (512, 150), (4, 70)])
def test_combine_matches_fp64_merge(devio, hd, ns):
    """The exported merge at every launch shape: four split groups (head_dim <= 512) or two
    (1024), 4, 8 or 16 splits in flight per thread, one pass or several (150 splits), split
    LSEs read lane-parallel beyond the first 64."""
    import torch
    import global_paged_gqa_amd as g
    rng = np.random.default_rng(5 + ns)
    B, H = 3, 5
    lse = rng.normal(0, 3, size=(B, H, ns)).astype(np.float32)
    lse[0, 0, :] = -np.inf
    lse[1, 2, [0, ns // 2, ns - 1]] = -np.inf
    o = (0.25 * rng.normal(size=(B, H, ns, hd))).astype(np.float32)   # attention-sized outputs
    o[lse == -np.inf] = np.nan          # empty splits must never be read
    out = torch.empty((B, H, hd), dtype=torch.int16, device="cuda")
    lo = torch.empty((B, H), dtype=torch.float32, device="cuda")
    g.gattn_combine(B, H, hd, ns, torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), out, lo)
    got_o = devio.host_bf16(out).astype(np.float64)
    got_l = lo.cpu().numpy()
    o64 = np.where(np.isfinite(lse)[..., None], o, 0.0).astype(np.float64)
    ref_o, ref_l = oracle.merge(lse.astype(np.float64), o64)
    assert got_l[0, 0] == -np.inf and np.all(got_o[0, 0] == 0)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    assert np.max(np.abs(got_l[fin] - ref_l[fin])) < 1e-5
    assert np.max(np.abs(got_o - ref_o)) < 1e-2


@pytest.mark.parametrize("n,hd", [(3, 512), (7, 512), (7, 1024), (7, 256)])
def test_combine_bits_independent_of_slot_count(devio, n, hd):
    """A (row, head)'s merged result is the same bit for bit whether its n splits sit in n slots
    or are padded with empty (-inf) slots up to 150, across every launch shape the slot count
    selects (thread groups 1, 2 or 4; 4, 8 or 16 loads in flight; one pass or several): the
    sums run in a fixed order and skip empty splits, so one row's output never depends on the
    batch's longest row. A NaN split LSE turns only its own (row, head) into NaN."""
    import torch
    import global_paged_gqa_amd as g
    rng = np.random.default_rng(11 + n)
    B, H = 2, 3
    lse = rng.normal(0, 3, size=(B, H, n)).astype(np.float32)
    o = (0.25 * rng.normal(size=(B, H, n, hd))).astype(np.float32)
    lse[1, 1, n - 1] = np.nan

    def run(ns):
        lp = np.full((B, H, ns), -np.inf, np.float32)
        op = np.full((B, H, ns, hd), np.nan, np.float32)
        lp[..., :n], op[..., :n, :] = lse, o
        out = torch.empty((B, H, hd), dtype=torch.int16, device="cuda")
        lo = torch.empty((B, H), dtype=torch.float32, device="cuda")
        g.gattn_combine(B, H, hd, ns, torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), out, lo)
        return out.cpu().numpy(), lo.cpu().numpy()

    base_o, base_l = run(n)
    assert np.all(np.isnan(devio.host_bf16(torch.from_numpy(base_o))[1, 1])) and np.isnan(base_l[1, 1])
    ok = np.ones((B, H), bool)
    ok[1, 1] = False
    assert np.all(np.isfinite(base_l[ok]))
    for ns in (5, 8, 12, 20, 30, 40, 70, 150):
        if ns < n:
            continue
        got_o, got_l = run(ns)
        assert np.array_equal(got_o[ok], base_o[ok]) and np.array_equal(got_l[ok], base_l[ok]), ns
        assert np.isnan(got_l[1, 1])


# ------------------------------------------------------------------------ head_dim 512 index probes
PROBE_L = 3000
PROBE_T = (0, 1, 15, 16, 32, 48, 64, 511, 512, 1023, 1024, 1025, 2047, 2048, 2559, 2560, PROBE_L - 17, PROBE_L - 16,
           PROBE_L - 1)


def _probe_batch(spec, t_star, key, n_filler=0, pt_stride=None, code_of=None):
    """Row 0 (L = PROBE_L): every query head is e_0, K[t*] = 200 e_0 and every other key 0, so at
    scale 1 every other weight underflows to exactly 0 and O must be V[t*] bit for bit. V[t*]
    holds a code of t* and the head dim (with K=V, V[t*] is K[t*]: the code sits in dims 1..hd-1
    beside the 200). Rows 1..n_filler are short random rows that only enlarge the grid."""
    L = [PROBE_L] + [1 + 7 * i for i in range(n_filler)]
    b = workloads.make_batch(spec, L, np.ones(len(L), np.int32), key, back="all", pt_stride=pt_stride)
    hd, P = spec.head_dim, spec.page_size
    b.q[0] = 0
    b.q[0, :, 0] = workloads.f32_to_bf16_bits(np.float32([1.0]))[0]
    code = workloads.f32_to_bf16_bits(np.float32(np.arange(hd) + 0.5 + (t_star % 97)))
    kk = np.zeros((PROBE_L, spec.num_kv_heads, hd), np.uint16)
    if spec.kv_shared:
        kk[t_star, :, :] = code
    kk[t_star, :, 0] = workloads.f32_to_bf16_bits(np.float32([200.0]))[0]
    pt = b.page_table[0]
    for t in range(PROBE_L):
        b.k_pool[pt[t // P], :, t % P, :] = kk[t]
        if not spec.kv_shared:
            b.v_pool[pt[t // P], :, t % P, :] = code if t == t_star else b.v_pool[pt[t // P], :, t % P, :]
    want = kk[t_star, 0] if spec.kv_shared else code
    return b, workloads.bf16_bits_to_f32(want).astype(np.float64)


HD512_SHAPES = {  # name: (kv_shared, split, filler rows, max_ctx, pt_stride) -> items = slots * 4 * rows
    "global-2waves-small": (False, 512, 0, None, None),      # 6 x 4 = 24 items
    "global-2waves": (False, 512, 1, 20000, 1250),           # 40 x 4 x 2 = 320 items
    "global-1wave": (False, 512, 8, 8192, 512),               # 16 x 4 x 9 = 576 items
    "kv-shared-4waves": (True, 1024, 0, None, None),         # 3 x 4 = 12 items
    "kv-shared-2waves": (True, 1024, 1, 40000, 2500),        # 40 x 4 x 2 = 320 items
    "kv-shared-1wave": (True, 1024, 8, 16384, 1024),         # 16 x 4 x 9 = 576 items
}


@pytest.mark.parametrize("shape", list(HD512_SHAPES))
def test_position_probe_hd512(devio, shape):
    """The position probe at head_dim 512 in each launch shape of the global family (with K = V a
    split's four page streams on four waves, on two waves of two streams, or on one wave in turn;
    with separate pools its two streams on two waves or on one), swept over page, split and stream
    edges: the output must be V[t*] bit for bit in every head."""
    shared, split, n_fill, max_ctx, pt_stride = HD512_SHAPES[shape]
    spec = workloads.LayerSpec("global", 32, 4, 512, kv_shared=shared, scale=1.0)
    for t_star in PROBE_T:
        b, want = _probe_batch(spec, t_star, (15, t_star, int(shared)), n_fill, pt_stride)
        d = devio.DeviceBatch(b)
        d.decode(split, max_ctx)
        out, _ = d.result()
        for h in range(spec.num_q_heads):
            assert np.array_equal(out[0, h], want), (shape, t_star, h)


@pytest.mark.parametrize("shared", [False, True], ids=["separate", "kv-shared"])
def test_position_probe_hd512_fp8(devio, shared):
    """The position probe over E4M3 pools at head_dim 512 (scales 1): K[t*] = 192 e_0 (an E4M3
    value), every other key code 0, and V[t*] (K[t*] with K=V) a code of t* and the dim; the
    output must be the widened V[t*] bit for bit."""
    spec = workloads.LayerSpec("global", 32, 4, 512, kv_shared=shared, scale=1.0)
    split = 1024 if shared else 512
    e4m3_192 = 0x74    # 1.5 * 2^7: exponent field 14 (bias 7), mantissa 0b100
    for t_star in PROBE_T:
        b, _ = _probe_batch(spec, t_star, (16, t_star, int(shared)))
        hd, P, Hkv = spec.head_dim, spec.page_size, spec.num_kv_heads
        # codes 0x08..0x57 (2^-6 .. 15, all finite) keyed by t* and the dim
        vcode = (8 + (np.arange(hd) + 3 * t_star) % 80).astype(np.uint8)
        k8 = np.zeros((PROBE_L, Hkv, hd), np.uint8)
        if shared:
            k8[t_star] = vcode
        k8[t_star, :, 0] = e4m3_192
        v8 = None if shared else np.zeros((PROBE_L, Hkv, hd), np.uint8)
        if not shared:
            v8[:] = 0x38   # 1.0 everywhere else
            v8[t_star] = vcode
        kp8 = np.zeros(b.k_pool.shape, np.uint8)
        vp8 = None if shared else np.zeros(b.k_pool.shape, np.uint8)
        pt = b.page_table[0]
        for t in range(PROBE_L):
            kp8[pt[t // P], :, t % P, :] = k8[t]
            if not shared:
                vp8[pt[t // P], :, t % P, :] = v8[t]
        b.fp8 = workloads.Fp8Kv(k8, k8 if shared else v8, kp8, vp8, 1.0, 1.0)
        want = oracle.e4m3_value((k8 if shared else v8)[t_star, 0])
        out, _ = devio.decode_fp8(b, split)
        for h in range(spec.num_q_heads):
            assert np.array_equal(out[0, h], want), (shared, t_star, h)
